// Host-side exhaustive check of the box geometry helpers shared by the HIP
// kernels: for every tile shape of volume 128 and every real extent of a box,
// the 128-bit real-slot mask equals the per-slot definition, and the box
// decoding matches the raster numbering of boxes. Prints "ok" on success.
#include <cstdio>

#include "../block_sparse_attention_13_amd/csrc/veda_internal.hpp"

int main() {
  using namespace veda;
  long checked = 0;
  for (int lt = 0; lt <= 7; ++lt)
    for (int lh = 0; lt + lh <= 7; ++lh) {
      const int lw = 7 - lt - lh;
      HeadGeo hg{uint8_t(lt), uint8_t(lh), uint8_t(lw), 0, 1, 1, 1, 1};
      for (int vt = 1; vt <= (1 << lt); ++vt)
        for (int vh = 1; vh <= (1 << lh); ++vh)
          for (int vw = 1; vw <= (1 << lw); ++vw) {
            BoxExtent e{0, 0, 0, vt, vh, vw};
            for (int base = 0; base < 128; base += 64) {
              const uint64_t m = box_slot_mask64(hg, e, base);
              for (int b = 0; b < 64; ++b) {
                const bool want = slot_is_real(hg, e, base + b);
                if (bool((m >> b) & 1ull) != want) {
                  std::printf("mismatch tile (%d,%d,%d) extent (%d,%d,%d) slot %d\n", 1 << lt, 1 << lh, 1 << lw,
                              vt, vh, vw, base + b);
                  return 1;
                }
                ++checked;
              }
            }
          }
    }
  // box decoding on a padded grid: boxes in raster order of box coordinates
  GeoTable g{};
  g.T = 21; g.H = 45; g.W = 80;
  HeadGeo hg{3, 2, 2, 0, 12, 20, 3 * 12 * 20, 1};  // tile (8,4,4)
  for (int tau = 0; tau < hg.nT; ++tau) {
    const BoxExtent e = box_extent(g, hg, tau);
    const int bt = tau / (12 * 20), by = (tau / 20) % 12, bx = tau % 20;
    if (e.t0 != 8 * bt || e.y0 != 4 * by || e.x0 != 4 * bx || e.vt != imin(8, 21 - 8 * bt) ||
        e.vh != imin(4, 45 - 4 * by) || e.vw != 4) {
      std::printf("box decode mismatch at %d\n", tau);
      return 1;
    }
  }
  std::printf("ok %ld slots\n", checked);
  return 0;
}
