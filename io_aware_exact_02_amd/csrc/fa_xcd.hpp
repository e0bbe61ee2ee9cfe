// Workgroup id -> (head, work item) so that each XCD's L2 serves few heads.
//
// The 256 compute units of the chip sit in eight XCDs, each with its own L2,
// and workgroup ids are handed to the XCDs round robin: id i runs on XCD
// i % 8, as the (i / 8)-th workgroup that XCD receives.  Every workgroup of a
// head reads the same K and V rows, so a head whose workgroups are spread
// over many XCDs is fetched from HBM into each of their L2s.
//
// The mapping splits heads and XCDs into G = gcd(BH, 8) matching groups:
// head bh belongs to group bh % G, XCD x to group x % G, each group holding
// a = BH / G heads and c = 8 / G XCDs.  Within a group the R items of its a
// heads are taken in windows of c consecutive items (heaviest first, as the
// kernels number them): the a * c (head, item) pairs of a window, in
// head-major order, are dealt out a to each XCD in XCD order.  So
//   * every XCD receives the same number of items per window, of about the
//     same weight, and the windows reach each XCD in item order;
//   * an XCD serves ceil(a / c) heads, or one more where a head straddles
//     two XCDs (BH = 12: two heads per XCD rather than the three that
//     bh = i % BH gives), and a head spans c / a XCDs, or one more;
//   * for BH a multiple of 8, or BH = 1, 2, 4, the mapping is bh = i % BH,
//     item = i / BH.
// When R is not a multiple of c, the last window holds ids that name no item
// (item >= R); those workgroups exit at once.
//
// Snake order (snake = true), for causal launches whose workgroups are all
// resident at once.  Then there is no dynamic dispatch to even out the
// causal work: an XCD hands its workgroups to its 32 compute units in
// passes, and with the heaviest items first every pass gives compute unit k
// an item about as heavy as the previous pass did, so the first units get
// the heaviest items of every pass.  Reversing every second full pass of 32
// pairs heavy with light.  A partial last pass keeps its order, so the
// mapping stays a bijection.  Launches with more workgroups than resident
// slots keep heaviest-first order, which dynamic dispatch balances.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct XcdItem {
  int bh;      // head (flattened batch * heads index)
  int item;    // work item of that head, 0 = heaviest
  bool valid;  // false: this id names no item
};

// Number of workgroup ids to launch for BH heads of R items each.
__host__ __device__ inline int64_t xcd_grid(int BH, int R) {
  if (BH <= 0 || R <= 0) return 0;
  const int G = (BH & -BH) < 8 ? (BH & -BH) : 8;
  const int a = BH / G;
  const int c = 8 / G;
  return static_cast<int64_t>(8) * a * ((R + c - 1) / c);
}

constexpr int kCusPerXcd = 32;  // 256 compute units in 8 XCDs

__host__ __device__ inline XcdItem xcd_item(uint32_t id, int BH, int R, bool snake = false) {
  const int G = (BH & -BH) < 8 ? (BH & -BH) : 8;  // gcd(BH, 8)
  const int a = BH / G;                            // heads per group
  const int c = 8 / G;                             // XCDs per group
  const int x = static_cast<int>(id & 7u);         // XCD
  int j = static_cast<int>(id >> 3);               // order on that XCD
  if (snake) {
    const int per_xcd = a * ((R + c - 1) / c);
    const int pass = j / kCusPerXcd;
    if ((pass & 1) != 0 && (pass + 1) * kCusPerXcd <= per_xcd)
      j = pass * kCusPerXcd + (kCusPerXcd - 1 - (j - pass * kCusPerXcd));
  }
  const int grp = x % G;
  const int xc = x / G;          // XCD's place within its group
  const int w = j / a;           // window
  const int flat = xc * a + (j - w * a);  // head-major place in the window
  const int hl = flat / c;
  XcdItem r;
  r.item = w * c + (flat - hl * c);
  r.bh = hl * G + grp;
  r.valid = r.item < R;
  return r;
}
