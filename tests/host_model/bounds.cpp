// Host model of the MMVQ kernels' memory accesses.
//
// Compiled for the host with QMV_HOST_MODEL, the kernels' own format and
// planning code (formats.hpp, plan.hpp) runs for every workgroup, team, lane
// and row of the launch the library would make, with loads replaced by
// bounds-checked host reads. Checks, for every case:
//   * every weight, header, scale and activation load lies inside its
//     buffer and is aligned as the device load requires, for q8_1
//     activations and for fp32 activations quantized in the prologue;
//   * every output row of every column is stored exactly once;
//   * the quantizer's and the block-dot kernel's loads stay in bounds.
// Prints one line per failing case and exits non-zero if any case fails.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "formats.hpp"
#include "mmq_plan.hpp"
#include "plan.hpp"

using namespace qmv;

static uint8_t* alloc16(size_t n) {
  // exactly n usable bytes at a 16-byte aligned address
  void* p = aligned_alloc(16, (n + 15) / 16 * 16 + 16);
  memset(p, 0x5A, (n + 15) / 16 * 16 + 16);
  return static_cast<uint8_t*>(p);
}

static int failures = 0;

static void begin(std::initializer_list<hostmodel::Range> rs) {
  hostmodel::ranges().assign(rs.begin(), rs.end());
  hostmodel::violations() = 0;
  hostmodel::accesses() = 0;
}

static void report(const char* what, bool ok_extra, const char* name, int64_t M, int64_t K, int nc, int g) {
  if (hostmodel::violations() != 0 || !ok_extra) {
    ++failures;
    printf("FAIL %s %s M=%lld K=%lld n=%d g=%d: %ld bad of %ld accesses%s\n", what, name, (long long)M,
           (long long)K, nc, g, hostmodel::violations(), hostmodel::accesses(), ok_extra ? "" : ", store coverage");
  }
}

// One launch of the rows kernel (plain G=1 or fused G=2), or of the id
// kernel for one expert (base = expert's matrix, tok = its token columns).
// passes: the team owns passes * R * P rows, taken R * P at a time.
template <class F>
static bool model_rows(const Shape& s, int R, int P, int G, int64_t M, const uint8_t* W, const uint8_t* Wg,
                       int64_t row_bytes, const uint8_t* y, int64_t ycol_bytes, const float* x, int64_t ldx,
                       const int* tok, int nc, std::vector<int>& stores, int passes = 1) {
  typename F::Wt wt;
  typename F::Act act;
  typename F::Dec dec;
  std::vector<int> seen(static_cast<size_t>(s.units) * P);   // active lanes per (slot, unit)
  for (int64_t b = 0; b < s.blocks; ++b) {
    for (int tl = 0; tl < s.teams_per_block; ++tl) {
      const int64_t team = b * s.teams_per_block + tl;
      std::fill(seen.begin(), seen.end(), 0);
      for (int lt = 0; lt < s.team_lanes; ++lt) {
        const Window w = team_window(team, lt, R * passes, P, s.units, M);
        const uint32_t slot_off = static_cast<uint32_t>(w.slot * row_bytes);
        // chunked rows: the lane's unit in each chunk, as the kernel walks them
        for (int c = 0; c < s.chunks; ++c) {
          bool active = w.active;
          const int unit = s.chunks == 1 ? w.unit : chunk_unit(lt, c, s.team_lanes, s.units, active);
          if (unit < 0 || unit >= s.units) return false;
          if (active) seen[static_cast<size_t>(w.slot) * s.units + unit] += 1;
          const typename F::Lane L = F::lane(unit);
          for (int pass = 0; pass < passes; ++pass) {
            const int64_t row0 = w.row0 + static_cast<int64_t>(pass) * R * P;
            const uint8_t* rp = W + row0 * row_bytes;
            const uint8_t* gp = Wg ? Wg + row0 * row_bytes : nullptr;
            for (int i = 0; i < R; ++i) {
              F::load_wt(wt, rp, slot_off, L);
              F::decode(wt, dec, L);
              rp += P * row_bytes;
              if (G == 2) {
                F::load_wt(wt, gp, slot_off, L);
                gp += P * row_bytes;
              }
            }
          }
          for (int j = 0; j < nc; ++j) {
            if (x) {
              typename F::XRaw xr;
              F::load_x(xr, x + tok[j] * ldx, unit);
              F::quant_x(act, xr);
            }
            else F::load_act(act, y + tok[j] * ycol_bytes, unit);
          }
        }
        // every unit of the row is some lane's in exactly one chunk
        if (s.chunks > 1 && lt == 0 && (static_cast<int64_t>(s.chunks) * s.team_lanes < s.units ||
                                        static_cast<int64_t>(s.chunks - 1) * s.team_lanes >= s.units))
          return false;
        if (lt == 0) {   // the store pattern of the team (one lane's view suffices)
          for (int pass = 0; pass < passes; ++pass) {
            const int64_t row0 = w.row0 + static_cast<int64_t>(pass) * R * P;
            const int64_t skip = w.skip - static_cast<int64_t>(pass) * R * P;
            for (int64_t i = 0; i < static_cast<int64_t>(R) * P; ++i) {
              if (i < skip) continue;
              const int64_t r = row0 + i;
              if (r < 0 || r >= M) return false;
              stores[r] += 1;
            }
          }
        }
      }
      // every unit of every slot's row is one active lane's
      for (int v : seen)
        if (v != 1) return false;
    }
  }
  return true;
}

// xpad < 0: q8_1 activations; else fp32 columns with ldx = K + xpad.
template <class F>
static void case_rows(const char* name, int64_t M, int64_t K, int nc, int g, int xpad = -1) {
  const int64_t row_bytes = K / F::kQK * F::kBlockBytes;
  const bool xf = xpad >= 0;
  const int64_t ldx = K + (xf ? xpad : 0);
  const int64_t ycol = K / 32 * kQ8Bytes;
  const int64_t act_bytes = xf ? ((nc - 1) * ldx + K) * 4 : nc * ycol;
  uint8_t* W = alloc16(M * row_bytes);
  uint8_t* Wg = g == 2 ? alloc16(M * row_bytes) : nullptr;
  uint8_t* y = alloc16(act_bytes);
  const float* x = xf ? reinterpret_cast<const float*>(y) : nullptr;
  const int units = static_cast<int>(K / F::kQK) * F::kUnitsPerBlock;
  const Shape s = plan_launch(M, units, launch_max_rows<F>(xf, nc, g), 256, launch_max_passes<F>(xf, nc, g), xf, nc, 0,
                              layout_depth_cap<F>(), rows_per_pass<F>(nc, g));
  // the launcher instantiates passes > 1 only at R = the register budget
  bool ok = s.team_lanes <= kLaunchBound && static_cast<int64_t>(s.rows) * s.slots * s.passes <= M &&
            (s.passes == 1 || ((s.passes == 2 || s.passes == 4) && s.rows == rows_per_pass<F>(nc, g))) &&
            (s.depth == 0 || (s.passes == 1 && s.depth < s.rows && (s.depth == 4 || s.depth == 8))) &&
            // chunked launches: as launch_rows_chunked instantiates them
            (s.chunks == 1 || (s.slots == 1 && s.passes == 1 && s.depth == 0 && s.teams_per_block == 1 &&
                               s.rows <= kChunkRows && s.rows <= rows_per_pass<F>(nc, g) &&
                               // the chunk count the kernel derives from units and TL
                               (s.units + s.team_lanes - 1) / s.team_lanes == s.chunks));
  int tok[kMaxCols];
  for (int j = 0; j < kMaxCols; ++j) tok[j] = j;
  std::vector<int> stores(M, 0);
  if (Wg) begin({{W, W + M * row_bytes}, {Wg, Wg + M * row_bytes}, {y, y + act_bytes}});
  else begin({{W, W + M * row_bytes}, {y, y + act_bytes}});
  ok = ok && model_rows<F>(s, s.rows, s.slots, g, M, W, Wg, row_bytes, xf ? nullptr : y, ycol, x, ldx, tok, nc,
                           stores, s.passes);
  for (int64_t r = 0; r < M && ok; ++r) ok = stores[r] == 1;
  report(xf ? "rows_f32" : "rows", ok, name, M, K, nc, g);
  free(W);
  free(Wg);
  free(y);
}

// id kernel: every expert with tokens reads its own matrix at e * stride.
template <class F>
static void case_id(const char* name, int64_t M, int64_t K, int E, int T, int g, int xpad = -1) {
  const int64_t row_bytes = K / F::kQK * F::kBlockBytes;
  const int64_t stride = (M * row_bytes + 15) / 16 * 16;
  const bool xf = xpad >= 0;
  const int64_t ldx = K + (xf ? xpad : 0);
  const int64_t ycol = K / 32 * kQ8Bytes;
  const int64_t act_bytes = xf ? ((T - 1) * ldx + K) * 4 : T * ycol;
  uint8_t* W = alloc16(E * stride);
  uint8_t* Wg = alloc16(E * stride);
  uint8_t* y = alloc16(act_bytes);
  const float* x = xf ? reinterpret_cast<const float*>(y) : nullptr;
  const int units = static_cast<int>(K / F::kQK) * F::kUnitsPerBlock;
  const int RB = id_block_rows<F>(g, xf);
  Shape s = plan_rows(M, units, RB, 256, QMV_TARGET_WAVES_PER_CU, 0);
  const int rb = s.chunks == 1 && static_cast<int64_t>(RB) * s.slots <= M ? RB : 1;   // as the launcher
  s.rows = rb;
  s.teams = (M + static_cast<int64_t>(rb) * s.slots - 1) / (static_cast<int64_t>(rb) * s.slots);
  s.blocks = (s.teams + s.teams_per_block - 1) / s.teams_per_block;
  begin({{W, W + E * stride}, {Wg, Wg + E * stride}, {y, y + act_bytes}});
  bool ok = true;
  for (int e = 0; e < E && ok; ++e) {
    int tok[kMaxCols];
    const int nt = T < kMaxCols ? T : kMaxCols;
    for (int j = 0; j < nt; ++j) tok[j] = (j + e) % T;
    std::vector<int> stores(M, 0);
    // rows per pass for nt tokens, as the kernel picks them
    const int rn = id_rows_n<F>(nt, rb, g, xf);
    ok = model_rows<F>(s, rn, s.slots, g, M, W + e * stride, g == 2 ? Wg + e * stride : nullptr, row_bytes,
                       xf ? nullptr : y, ycol, x, ldx, tok, nt, stores, rb / rn);
    for (int64_t q = 0; q < M && ok; ++q) ok = stores[q] == 1;
  }
  report(xf ? "id_f32" : "id", ok, name, M, K, T, g);
  free(W);
  free(Wg);
  free(y);
}

template <class F>
static void case_block_dots(const char* name, int64_t M, int64_t K, int nc) {
  const int64_t row_bytes = K / F::kQK * F::kBlockBytes;
  const int64_t nb = K / F::kQK;
  const int64_t ycol = K / 32 * kQ8Bytes;
  uint8_t* W = alloc16(M * row_bytes);
  uint8_t* y = alloc16(nc * ycol);
  begin({{W, W + M * row_bytes}, {y, y + nc * ycol}});
  typename F::Wt wt;
  typename F::Dec dec;
  int dots[F::kDotsPerBlock];
  for (int j = 0; j < nc; ++j)
    for (int64_t r = 0; r < M; ++r)
      for (int64_t b = 0; b < nb; ++b)
        for (int q = 0; q < F::kUnitsPerBlock; ++q) {
          const int u = static_cast<int>(b) * F::kUnitsPerBlock + q;
          const typename F::Lane L = F::lane(u);
          F::load_wt(wt, W + r * row_bytes, 0u, L);
          F::decode(wt, dec, L);
          F::int_dots(dec, y + j * ycol, u, dots);
        }
  report("block_dots", true, name, M, K, nc, 1);
  free(W);
  free(y);
}

// many-column (MFMA) kernel: every load of every lane, wave and step, in
// the workgroup-to-tile mapping the kernel uses; every output stored exactly
// once; every A load lands inside its row's LDS image (and the bytes the
// step's arithmetic reads are covered by loads of that step). G = 2: the
// gate/up form, whose gate loads must stay inside the gate matrix. XF: fp32
// columns (column stride K + 3), whose staged blocks must stay inside x and
// whose quantized blocks must write every byte of the B tiles exactly once.
template <class F, int RT, int CT, int NW, int G = 1, bool XF = false>
static void case_mmq(const char* name, int64_t M, int64_t K, int n) {
  using Gm = MmqGeom<F>;
  const int64_t row_bytes = K / F::kQK * F::kBlockBytes, ycol = K / 32 * kQ8Bytes;
  const int64_t ldx = K + 3, xfloats = (n - 1) * ldx + K;
  uint8_t* W = alloc16(M * row_bytes);
  uint8_t* Wg = G == 2 ? alloc16(M * row_bytes) : nullptr;
  uint8_t* y = XF ? nullptr : alloc16(n * ycol);
  uint8_t* x = XF ? alloc16(xfloats * 4) : nullptr;
  uint8_t* act = XF ? x : y;
  const int64_t act_bytes = XF ? xfloats * 4 : n * ycol;
  if (G == 2) begin({{W, W + M * row_bytes}, {Wg, Wg + M * row_bytes}, {act, act + act_bytes}});
  else begin({{W, W + M * row_bytes}, {act, act + act_bytes}});
  MmqArgs a{};
  a.W = W; a.Wg = Wg; a.y = y; a.M = M; a.row_bytes = row_bytes; a.ycol_bytes = ycol; a.n = n;
  a.x = reinterpret_cast<const float*>(x);
  a.ldx = ldx;
  a.nsb = static_cast<int>(K / 256);
  a.gx = static_cast<int>((M + 16 * RT - 1) / (16 * RT));
  a.gy = (n + 16 * CT - 1) / (16 * CT);
  const int64_t groups = static_cast<int64_t>(a.gx) * a.gy;
  std::vector<int> stores(M * n, 0);
  std::vector<int> tiles(groups, 0);
  bool ok = true;
  for (int64_t w = 0; w < groups && ok; ++w) {
    int64_t bx;
    int by;
    mmq_tile_of(w, a.gx, a.gy, bx, by);
    if (bx < 0 || bx >= a.gx || by < 0 || by >= a.gy) { ok = false; break; }
    tiles[bx * a.gy + by] += 1;
    const int64_t row_base = bx * 16 * RT;
    const int col_base = by * 16 * CT;
    for (int wave = 0; wave < NW; ++wave) {
      const int sb0 = mmq_sb_begin(a.nsb, wave, NW), sb1 = mmq_sb_begin(a.nsb, wave + 1, NW);
      for (int sb = sb0; sb < sb1; ++sb) {
        // bytes of each row image the step's loads write
        std::vector<std::vector<char>> img(16 * RT, std::vector<char>(Gm::kRowLds, 0));
        std::vector<char> btile(kMmqBPieces * 16 * CT, 0);
        for (int lane = 0; lane < 64; ++lane) {
          MmqOffsets<F, RT, CT> off;
          mmq_offsets<F, RT, CT>(a, row_base, col_base, lane, off);
          MmqStage<F, RT, CT, G, XF> st;
          mmq_stage_load<F, RT, CT, G, XF>(a, row_base, col_base, lane, sb, off, st);
          if constexpr (XF) {
            for (int j = 0; j < mmq_x_slots<CT>(); ++j) {
              int col, blk, c;
              mmq_x_pair(lane, j, 0, n, col, blk, c);
              const int at = col * 288 + blk * 36;
              if (col < 0 || col >= 16 * CT || at + 36 > kMmqBPieces * 16 * CT) {
                ok = false;
                continue;
              }
              for (int b = 0; b < 36; ++b) btile[at + b] += 1;
            }
          }
          for (int j = 0; j < mmq_a_slots<F, RT>(); ++j) {
            if (lane + kWave * j >= mmq_a_pieces<F>() * RT) continue;
            const int64_t ro = row_base * row_bytes + off.a[j];
            const int at = Gm::piece_lds(ro, sb, off.apc[j]);
            const int len = Gm::piece_short(off.apc[j]) ? 2 : 16;
            if (at < 0 || at + len > Gm::kRowLds || off.arow[j] >= 16 * RT) { ok = false; continue; }
            // the LDS image byte holds the super-block byte the kernel
            // expects there: source offset - image base = step byte
            const int64_t src = Gm::piece_src(ro, sb, off.apc[j]);
            const int64_t step0 = ro + static_cast<int64_t>(sb) * Gm::kStride;
            if (src - step0 != at - Gm::image_base(ro, sb)) ok = false;
            for (int b = 0; b < len; ++b) img[off.arow[j]][at + b] += 1;
          }
        }
        // every byte of every row's step (and, fp32 columns, of the B
        // tiles) is written exactly once
        for (size_t b = 0; XF && b < btile.size() && ok; ++b) ok = btile[b] == 1;
        for (int r = 0; r < 16 * RT && ok; ++r) {
          int64_t rr = row_base + r;
          rr = rr < M ? rr : M - 1;
          const int base = Gm::image_base((rr - row_base) * row_bytes + row_base * row_bytes, sb);
          const int step_bytes = static_cast<int>(K / F::kQK * F::kBlockBytes / a.nsb);
          for (int b = 0; b < step_bytes && ok; ++b) ok = img[r][base + b] == 1;
        }
      }
      for (int lane = 0; lane < 64; ++lane) {
        const int r16 = lane & 15, q = lane >> 4;
        for (int v = wave; v < RT * CT * 4; v += NW) {
          int64_t r;
          int c;
          mmq_store_pos<RT, CT>(v, q, r16, row_base, col_base, r, c);
          if (r < M && c < n) stores[c * M + r] += 1;
        }
      }
    }
  }
  for (int64_t i = 0; i < groups && ok; ++i) ok = tiles[i] == 1;
  for (int64_t i = 0; i < M * n && ok; ++i) ok = stores[i] == 1;
  report(XF ? (G == 2 ? "mmq_glu_f32" : "mmq_f32") : (G == 2 ? "mmq_glu" : "mmq"), ok, name, M, K, n, 1);
  free(W);
  free(Wg);
  free(y);
  free(x);
}

template <class F>
static void case_mmq_all(const char* name, int64_t M, int64_t K, int n) {
  case_mmq<F, 2, 2, 4>(name, M, K, n);
  case_mmq<F, 2, 2, 8>(name, M, K, n);
  case_mmq<F, 2, 1, 4>(name, M, K, n);
  case_mmq<F, 2, 1, 8>(name, M, K, n);
  case_mmq<F, 1, 1, 4>(name, M, K, n);
  case_mmq<F, 1, 1, 8>(name, M, K, n);
  case_mmq<F, 2, 2, 4, 2>(name, M, K, n);
  case_mmq<F, 2, 1, 8, 2>(name, M, K, n);
  case_mmq<F, 1, 1, 8, 2>(name, M, K, n);
  case_mmq<F, 2, 1, 4, 1, true>(name, M, K, n);
  case_mmq<F, 1, 1, 8, 1, true>(name, M, K, n);
  case_mmq<F, 2, 1, 8, 2, true>(name, M, K, n);
  case_mmq<F, 1, 1, 4, 2, true>(name, M, K, n);
}

// quantizer: 8 lanes per q8_1 block, 4 floats each (clamped to block 0 when
// past the end), column j at x + j*ldx
static void case_quantize(int64_t K, int64_t n, int64_t ldx) {
  const int64_t nb = K / 32;
  uint8_t* x = alloc16(((n - 1) * ldx + K) * 4);
  begin({{x, x + ((n - 1) * ldx + K) * 4}});
  const int64_t threads = (n * nb * 8 + 255) / 256 * 256;
  for (int64_t gid = 0; gid < threads; ++gid) {
    const int64_t blk = gid >> 3;
    const int sub = static_cast<int>(gid & 7);
    const int64_t bc = blk < n * nb ? blk : 0;
    const int64_t j = bc / nb, b = bc - j * nb;
    (void)ld_x4(x + 4 * (j * ldx + 32 * b + 4 * sub));
  }
  report("quantize", true, "q8_1", n, K, static_cast<int>(n), 1);
  free(x);
}

// Arguments: "full" adds the benchmark workloads; "small" runs a reduced
// case set (the build under the address and undefined-behaviour sanitizers).
int main(int argc, char** argv) {
  const bool full = argc > 1 && strcmp(argv[1], "full") == 0;
  const bool small = argc > 1 && strcmp(argv[1], "small") == 0;
  std::vector<int64_t> Ms = {1, 2, 3, 5, 7, 8, 9, 15, 16, 17, 31, 33, 64, 100, 129, 300, 1000};
  std::vector<int> nbs = {1, 2, 3, 5, 7, 8, 9, 16, 56};
  std::vector<int> ncs = {1, 2, 3, 4, 5, 6, 7, 8};
  if (small) {
    Ms = {1, 3, 17, 129};
    nbs = {1, 3, 16, 56};
    ncs = {1, 2, 8};
  }
  for (int64_t M : Ms) {
    for (int nb : nbs) {
      for (int nc : ncs) {
        for (int g = 1; g <= 2; ++g) {
          for (int xpad : {-1, 3}) {
            if (nb <= 16 || nc <= 2) {
              case_rows<Q4K>("q4_k", M, 256LL * nb, nc, g, xpad);
              case_rows<Q4K2>("q4_k2", M, 256LL * nb, nc, g, xpad);
              case_rows<Q6K>("q6_k", M, 256LL * nb, nc, g, xpad);
            }
            if (nb * 8 * 32 <= 16384 && (nb <= 16 || nc <= 2))
              case_rows<Q40>("q4_0", M, 32LL * nb * 8, nc, g, xpad);
            case_rows<Q40>("q4_0", M, 32LL * nb, nc, g, xpad);
            case_rows<Q80>("q8_0", M, 32LL * nb, nc, g, xpad);
            if (nb * 8 * 32 <= 16384 && (nb <= 16 || nc <= 2))
              case_rows<Q80>("q8_0", M, 32LL * nb * 8, nc, g, xpad);
          }
        }
      }
      if (M <= 64) {
        case_block_dots<Q4K>("q4_k", M, 256LL * nb, 2);
        case_block_dots<Q4K2>("q4_k2", M, 256LL * nb, 2);
        case_block_dots<Q6K>("q6_k", M, 256LL * nb, 2);
        case_block_dots<Q40>("q4_0", M, 32LL * nb, 2);
        case_block_dots<Q80>("q8_0", M, 32LL * nb, 2);
      }
    }
  }
  // longest rows a team holds without chunks
  for (int xpad : {-1, 1}) {
    case_rows<Q4K>("q4_k", 129, 16384, 1, 1, xpad);
    case_rows<Q4K2>("q4_k2", 129, 16384, 1, 1, xpad);
    case_rows<Q4K2>("q4_k2", 33, 32768, 1, 1, xpad);
    case_rows<Q4K2>("q4_k2", 33, 32768, 8, 2, xpad);
    case_rows<Q4K>("q4_k", 65, 16384, 8, 1, xpad);
    case_rows<Q4K2>("q4_k2", 65, 16384, 8, 1, xpad);
    case_rows<Q4K>("q4_k", 65, 16384, 1, 2, xpad);
    case_rows<Q4K2>("q4_k2", 65, 16384, 1, 2, xpad);
    case_rows<Q40>("q4_0", 129, 16384, 8, 2, xpad);
    case_rows<Q80>("q8_0", 129, 16384, 8, 2, xpad);
    case_rows<Q80>("q8_0", 33, 16384, 1, 1, xpad);
    case_rows<Q6K>("q6_k", 129, 32768, 1, 1, xpad);
    for (int g = 1; g <= 2; ++g) {
      case_id<Q4K>("q4_k", 200, 512, 4, 3, g, xpad);
      case_id<Q4K2>("q4_k2", 200, 512, 4, 3, g, xpad);
      case_id<Q4K>("q4_k", 300, 2048, 8, 8, g, xpad);
      case_id<Q4K2>("q4_k2", 300, 2048, 8, 8, g, xpad);
      case_id<Q40>("q4_0", 77, 1024, 5, 4, g, xpad);
      case_id<Q6K>("q6_k", 50, 768, 4, 2, g, xpad);
      case_id<Q4K>("q4_k", 1, 256, 3, 1, g, xpad);
      case_id<Q4K2>("q4_k2", 1, 256, 3, 1, g, xpad);
      for (int T : {1, 2, 3, 5, 8}) {
        case_id<Q4K>("q4_k", 77, 1024, 2, T, g, xpad);
        case_id<Q4K2>("q4_k2", 77, 1024, 2, T, g, xpad);
        case_id<Q6K>("q6_k", 33, 512, 2, T, g, xpad);
        case_id<Q40>("q4_0", 300, 512, 2, T, g, xpad);
        case_id<Q80>("q8_0", 45, 96, 3, T, g, xpad);
      }
    }
  }
  // rows longer than a team, walked in chunks (even and ragged last chunks)
  for (int xpad : {-1, 1}) {
    for (int nc : {1, 3, 8})
      for (int g = 1; g <= 2; ++g) {
        case_rows<Q4K2>("q4_k2", 37, 65536, nc, g, xpad);    // 1024 units: 2 chunks of 512
        case_rows<Q4K2>("q4_k2", 9, 33024, nc, g, xpad);     // 516 units: 2 chunks, 320-lane team
        case_rows<Q4K>("q4_k", 9, 16640, nc, g, xpad);       // 520 units
        case_rows<Q40>("q4_0", 37, 32768, nc, g, xpad);      // 1024 units
        case_rows<Q40>("q4_0", 5, 16416, nc, g, xpad);       // 513 units
        case_rows<Q80>("q8_0", 17, 40000, nc, g, xpad);      // 1250 units: 3 chunks
        case_rows<Q6K>("q6_k", 17, 65792, nc, g, xpad);      // 1028 units: 3 chunks
        case_rows<Q6K>("q6_k", 3, 33024, nc, g, xpad);       // 516 units
      }
    for (int g = 1; g <= 2; ++g)
      for (int T : {1, 3, 8}) {
        case_id<Q4K2>("q4_k2", 33, 65536, 3, T, g, xpad);
        case_id<Q40>("q4_0", 17, 32768, 2, T, g, xpad);
        case_id<Q6K>("q6_k", 9, 33024, 2, T, g, xpad);
        case_id<Q80>("q8_0", 5, 16416, 2, T, g, xpad);
      }
  }
  // the formats the pages name without layouts: Q4_1, Q5_0 (2-byte aligned
  // 22-byte blocks), Q5_1, Q5_K
  for (int64_t M : {1, 3, 17, 129})
    for (int nb : {1, 3, 16})
      for (int nc : {1, 2, 8})
        for (int g = 1; g <= 2; ++g)
          for (int xpad : {-1, 3}) {
            case_rows<Q41>("q4_1", M, 32LL * nb * 8, nc, g, xpad);
            case_rows<Q50>("q5_0", M, 32LL * nb, nc, g, xpad);
            case_rows<Q50>("q5_0", M, 32LL * nb * 8 + 32, nc, g, xpad);
            case_rows<Q51>("q5_1", M, 32LL * nb * 8, nc, g, xpad);
            case_rows<Q5K>("q5_k", M, 256LL * nb, nc, g, xpad);
          }
  for (int xpad : {-1, 1})
    for (int nc : {1, 8}) {
      case_rows<Q50>("q5_0", 9, 16416, nc, 2, xpad);     // chunked, ragged
      case_rows<Q41>("q4_1", 5, 32768, nc, 1, xpad);
      case_rows<Q5K>("q5_k", 7, 16640, nc, 2, xpad);     // 520 units
      for (int T : {1, 3, 8}) {
        case_id<Q41>("q4_1", 77, 1024, 3, T, 2, xpad);
        case_id<Q50>("q5_0", 33, 992, 2, T, 1, xpad);
        case_id<Q51>("q5_1", 17, 512, 2, T, 2, xpad);
        case_id<Q5K>("q5_k", 45, 768, 3, T, 2, xpad);
        case_id<Q5K>("q5_k", 9, 33024, 2, T, 1, xpad);   // chunked expert rows
      }
    }
  for (int64_t M : {1, 7, 33}) {
    case_block_dots<Q41>("q4_1", M, 96, 2);
    case_block_dots<Q50>("q5_0", M, 96, 2);
    case_block_dots<Q51>("q5_1", M, 96, 2);
    case_block_dots<Q5K>("q5_k", M, 512, 2);
  }
  // many-column kernel, a few shapes of every format (the full set below)
  for (int n : {9, 33}) {
    case_mmq_all<Q4K>("q4_k", 17, 512, n);
    case_mmq_all<Q6K>("q6_k", 33, 768, n);
    case_mmq_all<Q40>("q4_0", 17, 1280, n);
    case_mmq_all<Q80>("q8_0", 33, 512, n);
    case_mmq_all<Q41>("q4_1", 17, 768, n);
    case_mmq_all<Q50>("q5_0", 33, 512, n);
    case_mmq_all<Q51>("q5_1", 17, 1280, n);
    case_mmq_all<Q5K>("q5_k", 33, 768, n);
  }
  if (small) {
    printf("host model: %d failing case(s)\n", failures);
    return failures ? 1 : 0;
  }
  // teams that take their rows in passes (more rows wanted than a pass's
  // register budget), with a ragged last team
  for (int nc : {1, 2, 4, 5, 8})
    for (int g = 1; g <= 2; ++g)
      for (int xpad : {-1, 3}) {
        case_rows<Q4K>("q4_k", 3605, 14336, nc, g, xpad);
        case_rows<Q4K2>("q4_k2", 3605, 14336, nc, g, xpad);
        case_rows<Q6K>("q6_k", 3605, 14336, nc, g, xpad);
        case_rows<Q40>("q4_0", 3605, 14336, nc, g, xpad);
        case_rows<Q80>("q8_0", 3605, 14336, nc, g, xpad);
        case_rows<Q4K>("q4_k", 12301, 4096, nc, g, xpad);
        case_rows<Q40>("q4_0", 12301, 4096, nc, g, xpad);
        case_rows<Q80>("q8_0", 12301, 4096, nc, g, xpad);
        case_rows<Q6K>("q6_k", 12301, 4096, nc, g, xpad);
      }
  for (int64_t M : {1, 15, 16, 17, 33, 100})
    for (int64_t K : {256, 512, 768, 1024, 1280})
      for (int n : {6, 9, 16, 17, 33, 100}) {
        case_mmq_all<Q4K>("q4_k", M, K, n);
        case_mmq_all<Q6K>("q6_k", M, K, n);
        case_mmq_all<Q40>("q4_0", M, K, n);
        case_mmq_all<Q80>("q8_0", M, K, n);
        case_mmq_all<Q41>("q4_1", M, K, n);
        case_mmq_all<Q50>("q5_0", M, K, n);
        case_mmq_all<Q51>("q5_1", M, K, n);
        case_mmq_all<Q5K>("q5_k", M, K, n);
      }
  case_mmq<Q4K, 2, 2, 4>("q4_k", 300, 4096, 256);
  case_mmq<Q6K, 1, 1, 8>("q6_k", 300, 4096, 256);
  case_mmq<Q80, 2, 2, 8>("q8_0", 300, 4096, 256);
  for (int64_t K : {32, 64, 96, 1024, 14336})
    for (int64_t n : {1, 3, 8})
      for (int64_t pad : {0, 1, 3, 64}) case_quantize(K, n, K + pad);
  if (full) {   // the benchmark workloads
    for (int nc : {1, 2, 4, 8}) {
      case_rows<Q4K>("q4_k", 4096, 14336, nc, 1);
      case_rows<Q4K2>("q4_k2", 4096, 14336, nc, 1);
      case_rows<Q4K>("q4_k", 14336, 4096, nc, 1);
      case_rows<Q4K2>("q4_k2", 14336, 4096, nc, 1);
      case_rows<Q4K>("q4_k", 4096, 14336, nc, 1, 0);
      case_rows<Q4K2>("q4_k2", 4096, 14336, nc, 1, 0);
    }
    for (int nc : {2, 3, 4, 5}) {
      case_rows<Q4K>("q4_k", 14336, 4096, nc, 2);
      case_rows<Q4K>("q4_k", 14336, 4096, nc, 2, 0);
      case_rows<Q4K>("q4_k", 14336, 4096, nc, 1, 0);
      case_rows<Q80>("q8_0", 4096, 14336, nc, 1);
      case_rows<Q6K>("q6_k", 128256, 4096, nc, 1);
      case_rows<Q6K>("q6_k", 128256, 4096, nc, 1, 0);
    }
    case_rows<Q4K>("q4_k", 4096, 4096, 1, 1);
    case_rows<Q4K2>("q4_k2", 4096, 4096, 1, 1);
    case_rows<Q40>("q4_0", 256, 1024, 1, 1);
    case_rows<Q80>("q8_0", 4096, 14336, 1, 1);
    case_rows<Q80>("q8_0", 4096, 14336, 1, 1, 0);
    case_rows<Q6K>("q6_k", 128256, 4096, 1, 1);
    case_id<Q4K>("q4_k", 14336, 4096, 8, 8, 2);
    case_id<Q4K2>("q4_k2", 14336, 4096, 8, 8, 2);
    case_id<Q4K2>("q4_k2", 14336, 4096, 8, 8, 2, 0);
    case_mmq<Q4K, 2, 2, 4>("q4_k", 4096, 14336, 64);
    case_mmq<Q4K, 2, 1, 8>("q4_k", 4096, 14336, 16);
    case_mmq<Q4K, 1, 1, 8>("q4_k", 4096, 14336, 16);
    case_mmq<Q4K, 2, 2, 8>("q4_k", 14336, 4096, 32);
    case_mmq<Q6K, 2, 2, 4>("q6_k", 4096, 4096, 64);
    case_mmq<Q6K, 2, 1, 8>("q6_k", 2048, 4096, 16);
    case_mmq<Q41, 2, 1, 8>("q4_1", 4096, 14336, 16);
    case_mmq<Q50, 2, 1, 8>("q5_0", 4096, 14336, 16);
    case_mmq<Q51, 2, 2, 4>("q5_1", 4096, 14336, 32);
    case_mmq<Q5K, 2, 1, 8>("q5_k", 4096, 14336, 16);
    case_mmq<Q4K, 2, 1, 8, 2>("q4_k", 14336, 4096, 16);
    case_mmq<Q4K, 2, 2, 4, 2>("q4_k", 14336, 4096, 64);
    case_mmq<Q4K, 2, 1, 8, 1, true>("q4_k", 4096, 14336, 16);
    case_mmq<Q4K, 2, 1, 4, 1, true>("q4_k", 4096, 14336, 64);
    case_mmq<Q4K, 2, 1, 8, 2, true>("q4_k", 14336, 4096, 16);
    case_mmq<Q6K, 2, 1, 4, 1, true>("q6_k", 4096, 4096, 37);
    case_id<Q4K>("q4_k", 14336, 4096, 8, 8, 1);
    case_id<Q4K2>("q4_k2", 14336, 4096, 8, 8, 1);
  }
  printf("host model: %d failing case(s)\n", failures);
  return failures ? 1 : 0;
}
