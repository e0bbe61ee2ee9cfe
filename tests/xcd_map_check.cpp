// Host-side check of the workgroup -> (head, item) mapping in fa_xcd.hpp,
// compiled host-only by tests/test_xcd_map.py.
//
//   xcd_map_check dump BH R [snake]  print "id xcd bh item valid" for every id
//   xcd_map_check check       exhaustive checks for BH = 1..96, R = 1..80,
//                             plain and snake order;
//                             prints "ok <cases>" or the first failure
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <set>
#include <vector>

#include "fa_xcd.hpp"

static int fail(const char* what, int BH, int R, long id) {
  std::printf("FAIL %s BH=%d R=%d id=%ld\n", what, BH, R, id);
  return 1;
}

static int check_one(int BH, int R, bool snake) {
  const int64_t n = xcd_grid(BH, R);
  int G = 1;
  while (G < 8 && BH % (2 * G) == 0) G *= 2;
  const int a = BH / G, c = 8 / G;
  std::vector<int> seen(static_cast<size_t>(BH) * R, 0);
  std::vector<std::set<int>> heads_of_xcd(8), xcds_of_head(BH);
  std::vector<int> last_window(8, -1);
  std::vector<long> items_of_xcd(8, 0);
  for (int64_t id = 0; id < n; ++id) {
    const XcdItem t = xcd_item(static_cast<uint32_t>(id), BH, R, snake);
    if (t.bh < 0 || t.bh >= BH || t.item < 0) return fail("range", BH, R, id);
    if (t.item >= R) {
      if (t.valid) return fail("valid beyond R", BH, R, id);
      continue;
    }
    if (!t.valid) return fail("invalid below R", BH, R, id);
    if (seen[static_cast<size_t>(t.bh) * R + t.item]++) return fail("duplicate", BH, R, id);
    const int x = static_cast<int>(id % 8);
    heads_of_xcd[x].insert(t.bh);
    xcds_of_head[t.bh].insert(x);
    ++items_of_xcd[x];
    if (!snake) {
      // Items reach each XCD window by window (heaviest first).
      const int win = t.item / c;
      if (win < last_window[x]) return fail("window order", BH, R, id);
      last_window[x] = win;
      // BH a multiple of 8 or BH = 1, 2, 4: the plain i % BH mapping.
      if ((BH % 8 == 0 || 8 % BH == 0) && (t.bh != id % BH || t.item != id / BH))
        return fail("not i % BH", BH, R, id);
    }
  }
  for (size_t k = 0; k < seen.size(); ++k)
    if (seen[k] != 1) return fail("item missing", BH, R, static_cast<long>(k));
  // A window deals the head-major places [xc*a, (xc+1)*a) to the group's
  // XCD xc; place f belongs to the group's head f / c.
  for (int x = 0; x < 8; ++x) {
    const int xc = x / G;
    const int most = ((xc + 1) * a - 1) / c - (xc * a) / c + 1;
    if (static_cast<int>(heads_of_xcd[x].size()) > most) return fail("heads per xcd", BH, R, x);
  }
  for (int h = 0; h < BH; ++h) {
    const int hl = h / G;
    const int most = ((hl + 1) * c - 1) / a - (hl * c) / a + 1;
    if (static_cast<int>(xcds_of_head[h].size()) > most) return fail("xcds per head", BH, R, h);
  }
  // Full windows give every XCD the same count; the last window at most a
  // items more on some XCDs.
  long lo = items_of_xcd[0], hi = items_of_xcd[0];
  for (int x = 1; x < 8; ++x) {
    lo = items_of_xcd[x] < lo ? items_of_xcd[x] : lo;
    hi = items_of_xcd[x] > hi ? items_of_xcd[x] : hi;
  }
  if (hi - lo > a) return fail("balance", BH, R, hi - lo);
  return 0;
}

int main(int argc, char** argv) {
  if ((argc == 4 || argc == 5) && std::strcmp(argv[1], "dump") == 0) {
    const int BH = std::atoi(argv[2]), R = std::atoi(argv[3]);
    const bool snake = argc == 5 && std::strcmp(argv[4], "snake") == 0;
    const int64_t n = xcd_grid(BH, R);
    for (int64_t id = 0; id < n; ++id) {
      const XcdItem t = xcd_item(static_cast<uint32_t>(id), BH, R, snake);
      std::printf("%ld %ld %d %d %d\n", static_cast<long>(id), static_cast<long>(id % 8), t.bh,
                  t.item, t.valid ? 1 : 0);
    }
    return 0;
  }
  if (argc == 2 && std::strcmp(argv[1], "check") == 0) {
    int cases = 0;
    for (int snake = 0; snake < 2; ++snake)
      for (int BH = 1; BH <= 96; ++BH)
        for (int R = 1; R <= 80; ++R, ++cases)
          if (check_one(BH, R, snake != 0)) return 1;
    std::printf("ok %d\n", cases);
    return 0;
  }
  std::fprintf(stderr, "usage: xcd_map_check dump BH R | check\n");
  return 2;
}
