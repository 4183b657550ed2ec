// Work order of the large-tile grouped GEMM: which (M tile, N tile) workgroup L computes. Plain
// integer arithmetic, shared by the kernels and by a host-side check that enumerates every
// workgroup of a launch and confirms each tile is computed exactly once.
//
// The M tiles (entries of the tile table, in expert order) are cut into bands of band_rows_for(Nt)
// tiles, about 256 tiles per band, i.e. about one tile per CU. All XCDs work on the same band at
// the same time, so the band's routed rows and its experts' weights stay in the MALL. Inside a
// band the tiles are ordered in blocks: the band's N tiles are cut into 8 / gm groups and its M
// tiles into gm groups, the blocks are taken N group by N group, and a block is enumerated N-major.
// XCD x (workgroup L runs on XCD L % 8) takes the x-th eighth of that order, i.e. about one block
// of Nt * gm / 8 weight panels by band / gm row panels: the ~32 tiles its CUs run at once, which
// share their operands through the XCD's L2. A routed-row tile is then fetched into an XCD's L2
// by 8 / gm XCDs per band, an expert's weight panel by as many XCDs as M groups hold one of its
// tiles; band_groups_for picks gm. gm = 1 is a plain N-major order.
#pragma once

#if defined(__HIPCC__) || defined(__HIP__)
#define MOE_TO_HD __host__ __device__
#else
#define MOE_TO_HD
#endif

namespace moe {

// band height in M tiles: about 256 tiles per band
MOE_TO_HD inline int band_rows_for(int Nt) {
  const int b = (256 + Nt / 2) / Nt;
  return b < 4 ? 4 : (b > 16 ? 16 : b);
}

// M groups per band for Nt N tiles of bm-row M tiles over experts of about rows_per_expert rows.
// Experts of at most two tiles share a weight panel between at most two M tiles, so the grouping
// mostly decides how many XCDs fetch each routed-row tile: 4 M groups (2 N groups). Larger experts
// share their weight panels between the M tiles of a band, and a band's N-major order keeps those
// tiles on one XCD: 1 (measured: 4 M groups cut the GLM-5.2-shaped GEMM-1's fabric traffic by 16%, 2 raised the
// DeepSeek-V4-Pro-shaped share's by 15%; the kernel times did not move).
MOE_TO_HD inline int band_groups_for(int Nt, int bm, long long rows_per_expert) {
  (void)Nt;
  return rows_per_expert <= 2LL * bm ? 4 : 1;
}

// workgroups per XCD that a launch over at most max_mt M tiles and Nt N tiles needs: every
// XCD's share of each band (at most ceil(band tiles / 8)), and the surplus ones return at once
MOE_TO_HD inline int big_grid_per_xcd(int max_mt, int Nt) {
  return (max_mt * Nt + 7) / 8 + max_mt / band_rows_for(Nt) + 2;
}

// The tile of workgroup jx of XCD x over mt_total M tiles, Nt N tiles and gm M groups per band
// (1, 2, 4 or 8; anything else is taken as 1). False: no tile (a surplus workgroup). Over the
// workgroups jx < big_grid_per_xcd(mt_total, Nt) of every XCD, each tile goes to exactly one.
MOE_TO_HD inline bool big_tile_coords(int mt_total, int Nt, int gm, int x, int jx, int& ti,
                                      int& nt) {
  const int band_m = band_rows_for(Nt);
  const int nb_full = mt_total / band_m;
  const int tb_full = band_m * Nt;
  const int share_full = ((x + 1) * tb_full >> 3) - (x * tb_full >> 3);
  int band, band_rows, tb;
  if (jx < nb_full * share_full) {
    band = jx / share_full;
    jx -= band * share_full;
    band_rows = band_m;
    tb = tb_full;
  } else {
    jx -= nb_full * share_full;
    band = nb_full;
    band_rows = mt_total - nb_full * band_m;
    tb = band_rows * Nt;
    const int share_last = ((x + 1) * tb >> 3) - (x * tb >> 3);
    if (jx >= share_last) return false;
  }
  const int pos = (x * tb >> 3) + jx;  // < tb
  const int lgm = gm == 2 ? 1 : (gm == 4 ? 2 : (gm == 8 ? 3 : 0));
  const int lgn = 3 - lgm;
  // N group k holds N tiles [k Nt / 2^lgn, (k+1) Nt / 2^lgn) (rounded down) and positions
  // [nlo band_rows, nhi band_rows): the group of N index c = pos / band_rows
  const int c = pos / band_rows;
  const int k = (((c + 1) << lgn) - 1) / Nt;
  const int nlo = (k * Nt) >> lgn, nn = (((k + 1) * Nt) >> lgn) - nlo;
  // inside it, M group g holds M tiles [g band_rows / gm, (g+1) band_rows / gm) and local
  // positions [nn mlo, nn mhi): the group of M index i = r / nn; its block is N-major
  const int r = pos - nlo * band_rows;
  const int i = r / nn;
  const int g = (((i + 1) << lgm) - 1) / band_rows;
  const int mlo = (g * band_rows) >> lgm, mm = (((g + 1) * band_rows) >> lgm) - mlo;
  const int q = r - nn * mlo;
  nt = nlo + q / mm;
  ti = band * band_m + mlo + q % mm;
  return true;
}

}  // namespace moe
