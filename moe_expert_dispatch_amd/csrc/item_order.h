// Order of the grouped GEMM's work items (row tile, column tile): plain C++
// for the device and for host-side checks (the including file provides the
// __host__ / __device__ / __forceinline__ qualifiers).
#pragma once

namespace moe {

// Maps item w in [0, RT * CT) to (row tile, column tile). Items run through
// groups of GM row tiles x GN column tiles (row groups outermost); the last
// row group and the last column group of each row group take only the tiles
// that exist, so the numbering has no holes: with a static item-to-block
// assignment a hole would cost a block a whole item's time.
__host__ __device__ __forceinline__ void item_tile(int w, int RT, int CT, int GM, int GN,
                                                   int* rt, int* ct) {
  const int rg = w / (GM * CT);               // row group
  const int h = RT - rg * GM < GM ? RT - rg * GM : GM;  // its height
  const int v = w - rg * GM * CT;             // item inside the row group
  const int full = CT / GN;                   // whole column groups
  if (v < full * h * GN) {
    const int cg = v / (h * GN);
    const int within = v - cg * h * GN;
    *rt = rg * GM + within / GN;
    *ct = cg * GN + within % GN;
  } else {                                    // the last, narrower column group
    const int r = CT - full * GN;
    const int u = v - full * h * GN;
    *rt = rg * GM + u / r;
    *ct = full * GN + u % r;
  }
}

}  // namespace moe
