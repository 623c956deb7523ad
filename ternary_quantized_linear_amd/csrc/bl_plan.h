// bl_plan.h -- launch planning of the product kernels as plain host functions: which
// workgroups take which projection, rows, K segments and slices, and how much LDS and
// scratch that needs. No HIP types: the launchers (bl_gemv.hip, bl_skinny.hip,
// bl_prefill.hip, bl_bitdelta.hip) fill their kernel arguments from these plans, and a
// CPU test compiles this header alone and replays every plan's index arithmetic over
// many shapes (each row, chunk, segment and k-tile covered exactly once; LDS within a
// CU; 32-bit buffer offsets in range).
//
// Device figures enter as arguments (compute units, resident workgroups), so a plan is
// a pure function of the shapes and the part.
#pragma once
#include <stddef.h>
#include <stdint.h>

// The few index formulas that device code shares with the plans are compiled for both
// sides when this header is built by hipcc.
#if defined(__HIPCC__)
#define BL_PLAN_HD __host__ __device__
#else
#define BL_PLAN_HD
#endif

namespace bl {
namespace plan {

constexpr int kMaxGroup = 8;  // entries of one grouped launch (BL_MAX_GROUP)

// ---------------------------------------------------------------- decode GEMV
constexpr int kGemvWaves = 4;    // waves per workgroup (256 threads)
constexpr int kGemvMaxC = 512;   // 16-byte chunks per row: K <= 32768 (2-bit), 65536 (1-bit)

// Row mapping for C chunks of 16 bytes per row: L lanes per row (16, 32 or 64), I chunks
// per lane, S waves per row (their segments of CW chunks meet in LDS), RW = 64 / L rows
// per wave instruction; cfg numbers the kernel's instance of the sweep.
struct GemvCfg {
  int cfg, L, I, S, RW;
};

inline GemvCfg gemv_cfg(int C) {
  if (C <= 16) return {0, 16, 1, 1, 4};
  if (C <= 32) return {1, 32, 1, 1, 2};
  if (C <= 64) return {2, 64, 1, 1, 1};
  if (C <= 128) return {3, 64, 1, 2, 1};
  if (C <= 256) return {4, 64, 1, 4, 1};
  return {5, 64, 2, 4, 1};
}

struct GemvEntry {
  int src;      // index of the projection in the caller's list
  GemvCfg c;
  int N, C, CW;  // rows, chunks per row, chunks per wave segment
  int wg0, nwg;  // workgroups [wg0, wg0 + nwg)
};

struct GemvPlan {
  GemvEntry e[kMaxGroup];  // in dispatch order (costliest first)
  int count;
  int wgs;     // grid size
  int slots;   // 64-bit LDS combine words per workgroup (0 without segmented rows)
  bool big;    // some entry needs two chunks per lane (cfg 5)
};

// Relative cost of a byte streamed by segmented rows (S waves meet per row in LDS and an
// eighth of a segment's lanes may idle) against a byte of a one-wave row, in 1/16.
// Per-wave end times of the 8B layer (K = 14336 rows segmented, the others not) showed
// the segmented partition's waves ending ~2.4 us (median) before the others at 20/16;
// 18/16 and 19/16 measured 2-3% faster than 20/16 (alternating runs, two boxes).
constexpr int kGemvSegCost16 = 18;

// N[i], K[i]: the projections; codes: codes per 16-byte chunk (64 for 2-bit, 128 for
// 1-bit weights); resident: workgroups of the kernel the device keeps resident at once.
// One round of cap_num / cap_den of the resident workgroups, shared among the
// projections in proportion to their cost (at least one each, never one without a row
// group); the costliest partitions dispatch first; with weight_late, a partition's cost
// is raised by the fraction of the total dispatched before it (its waves get their first
// rows later).
inline GemvPlan gemv_plan(const int64_t* N, const int64_t* K, int count, int codes,
                          int resident, bool weight_late, int cap_num, int cap_den) {
  GemvPlan p{};
  int64_t cost[kMaxGroup], total = 0;
  int order[kMaxGroup];
  GemvCfg cfg[kMaxGroup];
  for (int i = 0; i < count; ++i) {
    cfg[i] = gemv_cfg((int)(K[i] / codes));
    p.big = p.big || cfg[i].cfg == 5;
    const int64_t bytes = N[i] * (K[i] / codes) * 16;
    cost[i] = cfg[i].S > 1 ? bytes * kGemvSegCost16 / 16 : bytes;
    total += cost[i];
    order[i] = i;
  }
  for (int i = 1; i < count; ++i)
    for (int j = i; j > 0 && cost[order[j]] > cost[order[j - 1]]; --j) {
      const int t = order[j];
      order[j] = order[j - 1];
      order[j - 1] = t;
    }
  int64_t wcost[kMaxGroup], wtotal = 0, before = 0;
  for (int o = 0; o < count; ++o) {
    const int64_t c = cost[order[o]];
    wcost[o] = weight_late ? c + (int64_t)((double)c * (double)before / (double)total) : c;
    before += c;
    wtotal += wcost[o];
  }
  const int cap = (int)((int64_t)resident * cap_num / cap_den);
  int wgs = 0, slots = 0;
  for (int o = 0; o < count; ++o) {
    const int i = order[o];
    GemvEntry& g = p.e[o];
    g.src = i;
    g.c = cfg[i];
    g.N = (int)N[i];
    g.C = (int)(K[i] / codes);
    g.CW = (g.C + g.c.S - 1) / g.c.S;
    const int groups = (g.N + g.c.RW - 1) / g.c.RW;
    const int gpw = kGemvWaves / g.c.S;
    int64_t n = (wcost[o] * (int64_t)(cap - count) + wtotal - 1) / wtotal;
    n = n < 1 ? 1 : n;
    const int64_t most = (groups + gpw - 1) / gpw;
    n = n > most ? most : n;
    g.nwg = (int)n;
    g.wg0 = wgs;
    wgs += g.nwg;
    if (g.c.S > 1) {  // one word per row group a workgroup visits
      const int64_t steps = (groups + n * gpw - 1) / (n * gpw);
      const int words = (int)(steps * gpw);
      slots = words > slots ? words : slots;
    }
  }
  p.count = count;
  p.wgs = wgs;
  p.slots = slots;
  return p;
}

// ---------------------------------------------------------------- skinny MFMA product
constexpr int kSkWaves = 8;                     // waves per workgroup (512 threads)
constexpr int kSkEntries = 2 * kMaxGroup;       // entries of one launch: projections x token slices
constexpr int kSkTileKB = 96;                   // LDS for the partial tiles, KiB
constexpr size_t kSkLdsMax = kSkTileKB * 1024 + 96 * 4 + 32 * 4;
constexpr int kSkLdsCU = 160 * 1024;            // LDS of one CU
constexpr size_t kSkRegroup = (size_t)kSkWaves * 16 * (64 * 7 + 16);  // per-wave regroup areas
static_assert(kSkLdsMax + 16 + kSkRegroup <= (size_t)kSkLdsCU, "LDS plan exceeds a CU");

struct SkEntry {
  int N, K;
  int nrb;       // row blocks of 16
  int mpw;       // a segment is 256 * mpw codes
  int nseg;      // segments covering K
  int S, teams;  // waves per team, teams per workgroup
  int npass;     // passes of a team over the segments
  int R;         // row blocks per team
  int wg0, nwg;
};

struct SkPlan {
  SkEntry e[kSkEntries];
  int count;
  int wgs;
  size_t tile_lds;  // LDS for tiles, counts and factors
  size_t lds;       // dynamic LDS of the launch (tiles, then the regroup areas)
  int wbase;        // byte offset of the regroup areas
  bool fits;        // tile LDS within kSkTileKB KiB (else the launch is refused)
};

// Segment length and team shape for K: the largest fraction of wave-steps spent on real
// codes (segments past K, idle waves and passes that leave waves without a segment
// count as waste); ties go to the longer segment, except that with one token block,
// rows needing several passes at 7 x 256 codes take segments of 512 codes when those
// waste no more (70B down, K = 28672, at 8 / 12 / 15 tokens: 19.2 / 19.9 / 21.4 us
// against 20.0 / 22.3 / 23.8 us in two passes of 7 x 256, the same at 2-4 tokens;
// segments of 256 codes were slower).
// TB: token blocks of 16 (1, 2 or 4); a wave holds 16 * mpw * TB registers of
// activations, so more token blocks take shorter segments (mpw <= 4 for two, <= 2 for
// four).
inline void sk_segments(int K, int TB, SkEntry& s) {
  const int c = K / 256;
  const int cand[4] = {7, 4, 2, 1};
  double best = -1.0;
  for (int m : cand) {
    if ((TB == 2 && m > 4) || (TB == 4 && m > 2)) continue;
    const int nseg = (c + m - 1) / m;
    const int S = nseg < kSkWaves ? nseg : kSkWaves;
    const int teams = kSkWaves / S;
    const int npass = (nseg + S - 1) / S;
    const double e = (double)teams * c / ((double)kSkWaves * m * npass);
    const bool multi = m == 2 && TB == 1 && s.mpw == 7 && s.npass > 1 && e > best - 1e-9;
    if (e > best + 1e-9 || multi) {
      best = e;
      s.mpw = m;
      s.nseg = nseg;
      s.S = S;
      s.teams = teams;
      s.npass = npass;
    }
  }
}

// cap: resident workgroups of the skinny kernel (one per CU with its LDS and registers);
// T[i]: tokens of entry i (entries of one launch may differ: token slices of one product). A workgroup of projection i with R row blocks per team reads
// R * teams * 16 rows of K/4 packed bytes from HBM and the T * K activation bytes of its
// segments (mostly L2 hits, weighted 1/4 per byte: timelines of the Llama-3-8B layer at
// T = 16 put the K = 14336 workgroups, with as many activation as weight bytes, ~1.7 us
// behind the others). The plan takes the smallest per-workgroup cost that one round of
// at most cap workgroups covers, never a workgroup without a row block, and more
// workgroups when a workgroup's tiles would not fit its LDS.
constexpr int64_t kSkActDiv = 4;

struct SkCost {
  int64_t rowbytes;  // weight bytes of one row block per team
  int64_t act;       // weighted activation bytes of one workgroup
  int64_t most;      // workgroups when every team has one row block
  int64_t need;      // fewest workgroups whose tiles fit the LDS
};

// Workgroups of entry s at per-workgroup cost tau (0 when tau is below one row block).
inline int64_t sk_wgs_at(const SkEntry& s, const SkCost& c, int64_t tau) {
  if (tau < c.act + c.rowbytes) return 0;
  int64_t r = (tau - c.act) / c.rowbytes;
  const int64_t rmax = (s.nrb + s.teams - 1) / s.teams;
  r = r < rmax ? r : rmax;
  int64_t n = (s.nrb + r * s.teams - 1) / (r * s.teams);
  return n < c.need ? c.need : n;
}

inline SkPlan skinny_plan(const int64_t* N, const int64_t* K, int count, int TB, int cap,
                          const int* T) {
  SkPlan p{};
  SkCost c[kSkEntries];
  int64_t lo = 0, hi = 0;
  for (int i = 0; i < count; ++i) {
    SkEntry& s = p.e[i];
    s.N = (int)N[i];
    s.K = (int)K[i];
    s.nrb = (s.N + 15) / 16;
    sk_segments(s.K, TB, s);
    c[i].rowbytes = (int64_t)s.teams * 16 * (K[i] / 4);
    c[i].act = (int64_t)T[i] * K[i] / kSkActDiv;
    c[i].most = (s.nrb + s.teams - 1) / s.teams;
    const int rcap = kSkTileKB / (s.teams * TB);
    c[i].need = (s.nrb + (int64_t)s.teams * rcap - 1) / ((int64_t)s.teams * rcap);
    const int64_t one = c[i].act + c[i].rowbytes;  // one row block per team
    const int64_t all = c[i].act + c[i].rowbytes * c[i].most;
    lo = one > lo ? one : lo;
    hi = all > hi ? all : hi;
  }
  // smallest tau in [lo, hi] whose workgroups fit one round (hi: the fewest workgroups)
  auto total = [&](int64_t tau) {
    int64_t t = 0;
    for (int i = 0; i < count; ++i) t += sk_wgs_at(p.e[i], c[i], tau);
    return t;
  };
  if (total(lo) > cap) {
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (total(mid) <= cap) hi = mid;
      else lo = mid + 1;
    }
  }
  int wgs = 0;
  size_t lds = 0;
  for (int i = 0; i < count; ++i) {
    SkEntry& s = p.e[i];
    int64_t n = sk_wgs_at(s, c[i], lo);
    const int64_t jmax = (s.nrb + n * s.teams - 1) / (n * s.teams);
    n = (s.nrb + jmax * s.teams - 1) / (jmax * s.teams);
    s.nwg = (int)n;
    s.R = (int)jmax;
    s.wg0 = wgs;
    wgs += s.nwg;
    const size_t need = (size_t)s.teams * s.R * (TB * 1024 + 4) + 16 * TB * sizeof(float);
    lds = need > lds ? need : lds;
  }
  p.count = count;
  p.wgs = wgs;
  p.tile_lds = lds;
  p.fits = lds <= kSkLdsMax;
  p.wbase = (int)((lds + 15) / 16 * 16);
  p.lds = (size_t)p.wbase + kSkRegroup;
  return p;
}

// ---------------------------------------------------------------- tiled GEMM, split K
constexpr int kPfKT = 128;  // codes per k-tile

// K slices for a product of T <= 128 tokens on 32*MI x 256 tiles: as many as give every
// CU about one workgroup, keeping at least 8 k-tiles per slice; 1 when the tiles alone
// fill the device (or T > 128, or K not a whole number of k-tiles).
inline int splitk_slices(int T, int N, int K, int cus) {
  if (T > 128 || K % kPfKT) return 1;
  const int MI = (T + 31) / 32;
  const int64_t tiles = (int64_t)((T + 32 * MI - 1) / (32 * MI)) * ((N + 255) / 256);
  if (tiles >= cus) return 1;
  int P = (int)((cus + tiles - 1) / tiles);
  const int most = (K / kPfKT) / 8;
  P = P < most ? P : most;
  return P < 1 ? 1 : P;
}

// The launch of P requested slices: ktn k-tiles per slice and the slices actually used
// (no empty slice).
struct SplitK {
  int ktn, P;
};

inline SplitK splitk_shape(int K, int P) {
  const int nkt = K / kPfKT;
  SplitK s;
  s.ktn = (nkt + P - 1) / P;
  s.P = (nkt + s.ktn - 1) / s.ktn;
  return s;
}

inline size_t splitk_scratch_bytes(int T, int N, int K, int cus) {
  const int P = splitk_slices(T, N, K, cus);
  return P > 1 ? (size_t)P * T * N * sizeof(int32_t) : 0;
}

// Workgroups of a tiled launch are numbered XCD-major (workgroup b runs on XCD b % 8):
// logical tile (b % 8) * per_xcd + b / 8, with per_xcd = ceil(tiles / 8) and a grid of
// 8 * per_xcd (indices past the tiles return at once).
inline int xcd_per(int64_t tiles) { return (int)((tiles + 7) / 8); }
BL_PLAN_HD inline int xcd_tile(int bid, int per_xcd) { return (bid & 7) * per_xcd + (bid >> 3); }

// ---------------------------------------------------------------- BitDelta
constexpr int kBdWaves = 8;
constexpr int kBdMaxB = 8;
constexpr size_t kBdLdsMax = 64 * 1024;

// LDS per workgroup: the row partials [R][S][kBdMaxB], one slot per row, wave and model.
constexpr size_t bd_lds_bytes(int R, int S) {
  return (size_t)R * S * kBdMaxB * sizeof(float);
}

// Workgroups (returned) and rows per workgroup (*R) for N rows: one resident round
// (cap), or more when a workgroup's row slots would not fit its LDS; then as few
// workgroups as give the same number of rows each.
inline int bd_plan(int64_t N, int S, int cap, int* R) {
  const int64_t rmax = (int64_t)(kBdLdsMax / bd_lds_bytes(1, S));
  int64_t nwg = cap < N ? cap : N;
  int64_t r = (N + nwg - 1) / nwg;
  if (r > rmax) r = rmax;
  nwg = (N + r - 1) / r;
  *R = (int)((N + nwg - 1) / nwg);
  return (int)nwg;
}

}  // namespace plan
}  // namespace bl
