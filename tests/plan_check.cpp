// plan_check.cpp -- replays the launch plans of bl_plan.h on the CPU (built and run by
// tests/test_launch_plans.py). For each shape it walks the index arithmetic each kernel
// applies to its plan -- which rows, 16-byte chunks, row blocks, K segments, K slices and
// tiles every workgroup and wave takes -- and checks that each is covered exactly once,
// that LDS stays within a CU and that buffer offsets fit their 32-bit fields. Prints one
// line per failed check and exits non-zero on any.
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../ternary_quantized_linear_amd/csrc/bl_plan.h"

using namespace bl::plan;

static long g_cases = 0, g_fail = 0;

#define CHECK(cond, ...)                \
  do {                                  \
    if (!(cond)) {                      \
      ++g_fail;                         \
      if (g_fail < 40) {                \
        printf("FAIL %s: ", #cond);     \
        printf(__VA_ARGS__);            \
        printf("\n");                   \
      }                                 \
    }                                   \
  } while (0)

// ---------------------------------------------------------------- GEMV
// The kernel's sweep (bl_gemv.hip): wave `wave` of partition workgroup wgl takes segment
// wave % S of row groups g0 = wgl * GPW + wave / S, g0 + stride, ... (stride = nwg * GPW,
// GPW = 4 / S) up to the last group; lane (sub = lane / L, jl = lane % L) reads chunk
// cbase + jl + L * i (i < I) of row g * RW + sub when jl + L * i < CW and the chunk is
// inside the row; combine word k * GPW + wave / S for the k-th group it visits.
static void check_gemv(const int64_t* N, const int64_t* K, int count, int codes, int resident,
                       bool late) {
  ++g_cases;
  // the 2-bit launch takes 5/8 of the resident workgroups (1/2 with rows of more than
  // 256 chunks), the 1-bit one half
  bool big = false;
  for (int i = 0; i < count; ++i) big = big || gemv_cfg((int)(K[i] / codes)).cfg == 5;
  const bool q = codes == 64 && !big;
  const GemvPlan p = gemv_plan(N, K, count, codes, resident, late, q ? 5 : 1, q ? 8 : 2);
  CHECK(p.count == count, "count");
  int next = 0;
  bool seen[kMaxGroup] = {};
  for (int o = 0; o < count; ++o) {
    const GemvEntry& e = p.e[o];
    CHECK(e.src >= 0 && e.src < count && !seen[e.src], "entry %d src %d", o, e.src);
    seen[e.src] = true;
    CHECK(e.N == N[e.src] && (int64_t)e.C * codes == K[e.src], "entry %d shape", o);
    CHECK(e.wg0 == next && e.nwg >= 1, "entry %d workgroups %d+%d", o, e.wg0, e.nwg);
    next = e.wg0 + e.nwg;
    const GemvCfg c = e.c;
    CHECK(c.L * c.RW == 64 && 4 % c.S == 0, "cfg");
    CHECK(e.C <= kGemvMaxC, "C %d", e.C);
    CHECK((int64_t)c.S * e.CW >= e.C && (int64_t)c.L * c.I >= e.CW, "segments C %d CW %d", e.C,
          e.CW);
    const int GPW = kGemvWaves / c.S;
    const int64_t stride = (int64_t)e.nwg * GPW;
    const int64_t ngroups = (e.N + c.RW - 1) / c.RW;
    CHECK((int64_t)(e.nwg - 1) * GPW < ngroups, "entry %d: a workgroup without a row group", o);
    std::vector<unsigned char> hit((size_t)e.N * e.C, 0);
    for (int wgl = 0; wgl < e.nwg; ++wgl)
      for (int wave = 0; wave < kGemvWaves; ++wave) {
        const int64_t g0 = (int64_t)wgl * GPW + wave / c.S;
        if (g0 >= ngroups) continue;
        const int64_t glast = g0 + ((ngroups - 1 - g0) / stride) * stride;
        const int s = wave % c.S, cbase = s * e.CW;
        for (int64_t g = g0, k = 0; g <= glast; g += stride, ++k) {
          if (c.S > 1) CHECK(k * GPW + wave / c.S < p.slots, "combine word past %d", p.slots);
          for (int sub = 0; sub < c.RW; ++sub) {
            const int64_t row = g * c.RW + sub;
            if (row >= e.N) continue;
            for (int jl = 0; jl < c.L; ++jl)
              for (int i = 0; i < c.I; ++i) {
                const int ch = jl + c.L * i;
                if (ch < e.CW && cbase + ch < e.C) {
                  unsigned char& h = hit[(size_t)row * e.C + cbase + ch];
                  h = (unsigned char)(h + 1);
                }
              }
          }
        }
      }
    size_t bad = 0;
    for (unsigned char h : hit) bad += h != 1;
    CHECK(bad == 0, "entry %d (N %d, K %lld): %zu chunks not covered exactly once", o, e.N,
          (long long)K[e.src], bad);
    // chunk byte offsets are 32-bit per lane
    CHECK((int64_t)16 * e.C < (int64_t(1) << 32), "chunk offset");
  }
  CHECK(p.wgs == next, "grid %d vs %d", p.wgs, next);
  CHECK((size_t)p.slots * 8 <= 64 * 1024, "combine words %d exceed 64 KiB", p.slots);
  // the kernel's LDS: the combine words, then one prepared-activation record and a sum
  // per chunk of the longest row (64 + 4 bytes for 2-bit chunks, 128 + 4 for 1-bit)
  int64_t maxC = 0;
  for (int i = 0; i < count; ++i) maxC = K[i] / codes > maxC ? K[i] / codes : maxC;
  const size_t lds = (((size_t)p.slots * 8 + 15) & ~(size_t)15) + (size_t)(codes + 4) * maxC;
  CHECK(lds <= 160 * 1024, "GEMV LDS %zu exceeds a CU", lds);
}

// ---------------------------------------------------------------- skinny
// The kernel (bl_skinny.hip): team tg = wgl * teams + team of TT = nwg * teams takes row
// blocks rb = tg + fr * TT (fr < R); wave seg of a team takes segment p * S + seg in pass
// p < npass; a segment is 256 * mpw codes of K.
static void check_skinny(const int64_t* N, const int64_t* K, int count, int TB, int cap,
                         const int* Ts) {
  ++g_cases;
  const SkPlan p = skinny_plan(N, K, count, TB, cap, Ts);
  int next = 0;
  for (int i = 0; i < count; ++i) {
    const SkEntry& e = p.e[i];
    CHECK(e.wg0 == next && e.nwg >= 1, "entry %d workgroups", i);
    next = e.wg0 + e.nwg;
    CHECK(e.S >= 1 && e.S * e.teams <= kSkWaves, "team shape S %d teams %d", e.S, e.teams);
    CHECK(e.mpw == 1 || e.mpw == 2 || (e.mpw == 4 && TB <= 2) || (e.mpw == 7 && TB == 1),
          "mpw %d", e.mpw);
    CHECK((int64_t)e.nseg * e.mpw * 256 >= K[i] && (int64_t)(e.nseg - 1) * e.mpw * 256 < K[i],
          "segments of K %lld", (long long)K[i]);
    CHECK(e.npass * e.S >= e.nseg && (e.npass - 1) * e.S < e.nseg, "passes");
    std::vector<int> segs(e.nseg, 0);
    for (int pp = 0; pp < e.npass; ++pp)
      for (int s = 0; s < e.S; ++s)
        if (pp * e.S + s < e.nseg) segs[pp * e.S + s]++;
    for (int v : segs) CHECK(v == 1, "segment coverage");
    const int64_t TT = (int64_t)e.nwg * e.teams;
    std::vector<int> rbs(e.nrb, 0);
    for (int64_t tg = 0; tg < TT; ++tg)
      for (int fr = 0; fr < e.R; ++fr) {
        const int64_t rb = tg + fr * TT;
        if (rb < e.nrb) rbs[rb]++;
      }
    size_t bad = 0;
    for (int v : rbs) bad += v != 1;
    CHECK(bad == 0, "entry %d (N %lld, K %lld): %zu row blocks not covered once", i,
          (long long)N[i], (long long)K[i], bad);
    CHECK((int64_t)(e.nwg - 1) * e.teams < e.nrb, "a workgroup without a row block");
    // 32-bit buffer ranges: activations T*K, outputs T*N*4, a row block 16 rows of K/4
    const int T = Ts[i];
    CHECK(T >= 1 && T <= 16 * TB, "entry %d: %d tokens in %d token blocks", i, T, TB);
    CHECK((int64_t)T * K[i] < (int64_t(1) << 32), "activation range");
    CHECK((int64_t)T * N[i] * 4 < (int64_t(1) << 31), "output range");
    CHECK((int64_t)16 * (K[i] / 4) < (int64_t(1) << 31), "weight range");
  }
  CHECK(p.wgs == next, "grid");
  // one round of resident workgroups unless the tiles' LDS alone asks for more
  int64_t fewest = 0;
  for (int i = 0; i < count; ++i) {
    const SkEntry& e = p.e[i];
    const int rcap = kSkTileKB / (e.teams * TB);
    const int64_t need = (e.nrb + (int64_t)e.teams * rcap - 1) / ((int64_t)e.teams * rcap);
    fewest += need > 1 ? need : 1;
  }
  if (fewest <= cap) CHECK(p.wgs <= cap, "grid %d exceeds %d resident workgroups", p.wgs, cap);
  if (p.fits) {
    CHECK(p.tile_lds <= kSkLdsMax, "tile LDS %zu", p.tile_lds);
    CHECK(p.lds <= (size_t)kSkLdsCU, "LDS %zu exceeds a CU", p.lds);
    CHECK(p.wbase % 16 == 0 && (size_t)p.wbase >= p.tile_lds, "regroup base");
  }
}

// ---------------------------------------------------------------- split K and tiles
static void check_splitk(int T, int N, int K, int cus) {
  ++g_cases;
  const int P = splitk_slices(T, N, K, cus);
  CHECK(P >= 1, "P");
  if (T > 128 || K % kPfKT) {
    CHECK(P == 1, "no split beyond 128 tokens or for ragged K");
    return;
  }
  const int nkt = K / kPfKT;
  if (P > 1) CHECK(nkt / P >= 8, "slices of at least 8 k-tiles (T %d N %d K %d P %d)", T, N, K, P);
  const SplitK s = splitk_shape(K, P);
  CHECK(s.P >= 1 && s.P <= P && s.ktn >= 1, "shape");
  std::vector<int> kt(nkt, 0);
  for (int sl = 0; sl < s.P; ++sl) {
    const int kb = sl * s.ktn, n = (s.ktn < nkt - kb ? s.ktn : nkt - kb);
    CHECK(n >= 1, "empty slice");
    for (int k = kb; k < kb + n; ++k) kt[k]++;
  }
  for (int v : kt) CHECK(v == 1, "k-tile coverage");
  const size_t need = s.P > 1 ? (size_t)s.P * T * N * 4 : 0;
  CHECK(need <= splitk_scratch_bytes(T, N, K, cus), "scratch");
  // the allocation-free entry point's 64 MiB covers every split on this part
  if (cus <= 304) CHECK(splitk_scratch_bytes(T, N, K, cus) <= ((size_t)64 << 20), "scratch > 64 MiB");
  // XCD-major numbering: every logical tile from exactly one workgroup
  const int MI = (T + 31) / 32;
  const int64_t tiles = (int64_t)((T + 32 * MI - 1) / (32 * MI)) * ((N + 255) / 256) * s.P;
  const int per = xcd_per(tiles);
  std::vector<int> seen(8 * (size_t)per, 0);
  for (int bid = 0; bid < 8 * per; ++bid) {
    const int t = xcd_tile(bid, per);
    CHECK(t >= 0 && t < 8 * per, "tile index");
    if (t >= 0 && t < 8 * per) seen[t]++;
  }
  for (int64_t t = 0; t < tiles; ++t) CHECK(seen[t] == 1, "tile %lld", (long long)t);
}

static void check_bitdelta(int64_t N, int M, int cap) {
  ++g_cases;
  const int S = (M + 1023) / 1024;
  int R = 0;
  const int nwg = bd_plan(N, S, cap, &R);
  CHECK(nwg >= 1 && R >= 1, "plan");
  CHECK((int64_t)nwg * R >= N && (int64_t)(nwg - 1) * R < N, "rows N %lld", (long long)N);
  CHECK(bd_lds_bytes(R, S) <= kBdLdsMax, "LDS N %lld M %d R %d", (long long)N, M, R);
}

int main() {
  const int residents[] = {256 * 8, 256 * 4, 256 * 2, 304 * 8, 80 * 8};
  const int64_t rows[] = {1, 3, 4, 16, 17, 100, 1000, 1001, 1024, 4096, 4097, 6144, 8192, 14336, 28672};
  // GEMV, one projection: every chunk count the kernel takes (K % 64 == 0, K <= 32768)
  const int64_t gks[] = {64, 128, 576, 1024, 1088, 2048, 4096, 4160, 8192, 8256, 14336, 16384, 16448, 28672, 32768};
  for (int r : residents)
    for (int64_t n : rows)
      for (int64_t k : gks) {
        if (n * k > (int64_t)40000000 && r != residents[0]) continue;  // bound the run time
        check_gemv(&n, &k, 1, 64, r, true);
      }
  // the 1-bit form (128 codes per chunk)
  for (int64_t n : rows)
    for (int64_t k : gks) {
      const int64_t k2 = 2 * k;
      check_gemv(&n, &k2, 1, 128, residents[0], false);
    }
  // grouped launches: the seven projections of a Llama-3-8B layer, its fused four, and
  // ragged mixes
  {
    const int64_t N7[] = {4096, 1024, 1024, 4096, 14336, 14336, 4096};
    const int64_t K7[] = {4096, 4096, 4096, 4096, 4096, 4096, 14336};
    const int64_t N4[] = {6144, 4096, 28672, 4096};
    const int64_t K4[] = {4096, 4096, 4096, 14336};
    const int64_t Nm[] = {17, 1001, 3, 4097, 100, 65, 2, 31};
    const int64_t Km[] = {64, 4160, 32768, 128, 14336, 1088, 576, 8192};
    for (int r : residents) {
      check_gemv(N7, K7, 7, 64, r, true);
      check_gemv(N4, K4, 4, 64, r, true);
      check_gemv(Nm, Km, 8, 64, r, true);
      const int64_t K7b[] = {8192, 8192, 8192, 8192, 8192, 8192, 28672};
      check_gemv(N7, K7b, 7, 128, r, false);
    }
  }
  // skinny: K % 256 == 0 up to BL_MAX_K, 1 or 2 token blocks, a few device sizes
  const int caps[] = {256, 304, 80};
  const int64_t sks[] = {256, 512, 1024, 1792, 2304, 4096, 8192, 14336, 16384, 28672, 65536, 131840};
  for (int cap : caps)
    for (int TB = 1; TB <= 4; TB *= 2)
      for (int64_t n : rows)
        for (int64_t k : sks)
          for (int T : {8 * TB + 1, 16 * TB}) check_skinny(&n, &k, 1, TB, cap, &T);
  {
    const int64_t N7[] = {4096, 1024, 1024, 4096, 14336, 14336, 4096};
    const int64_t K7[] = {4096, 4096, 4096, 4096, 4096, 4096, 14336};
    const int64_t N4[] = {6144, 4096, 28672, 4096};
    const int64_t K4[] = {4096, 4096, 4096, 14336};
    const int64_t Nm[] = {1, 16, 17, 1000, 28672, 3, 65535, 8192};
    const int64_t Km[] = {256, 131840, 512, 14336, 8192, 28672, 256, 28672};
    for (int cap : caps)
      for (int TB = 1; TB <= 4; TB *= 2)
        for (int T : {8 * TB + 1, 16 * TB}) {
          const int Ts[8] = {T, T, T, T, T, T, T, T};
          check_skinny(N7, K7, 7, TB, cap, Ts);
          check_skinny(N4, K4, 4, TB, cap, Ts);
          check_skinny(Nm, Km, 8, TB, cap, Ts);
        }
    // token slices of one product as entries of one launch: the first slices full, the
    // last one ragged (as the launcher cuts 17..64 tokens)
    for (int cap : caps)
      for (int TB = 1; TB <= 2; TB *= 2)
        for (int last : {1, 8 * TB + 3, 16 * TB})
          for (int parts = 2; parts <= 4; ++parts) {
            int64_t Ns[8], Ks[8];
            int Ts[8];
            for (int j = 0; j < parts; ++j) {
              Ns[j] = N4[2];
              Ks[j] = K4[2];
              Ts[j] = j + 1 < parts ? 16 * TB : last;
              Ns[parts + j] = N4[3];
              Ks[parts + j] = 28672;
              Ts[parts + j] = Ts[j];
            }
            check_skinny(Ns, Ks, parts, TB, cap, Ts);
            check_skinny(Ns, Ks, 2 * parts, TB, cap, Ts);
          }
    // the seven projections of a layer in two slices each: sixteen entries at most
    for (int cap : caps)
      for (int last : {1, 9, 16}) {
        int64_t Ns[16], Ks[16];
        int Ts[16];
        for (int j = 0; j < 14; ++j) {
          Ns[j] = N7[j / 2];
          Ks[j] = K7[j / 2];
          Ts[j] = j % 2 ? last : 16;
        }
        Ns[14] = Nm[3]; Ks[14] = Km[3]; Ts[14] = 16;
        Ns[15] = Nm[6]; Ks[15] = Km[6]; Ts[15] = last;
        check_skinny(Ns, Ks, 14, 1, cap, Ts);
        check_skinny(Ns, Ks, 16, 1, cap, Ts);
      }
  }
  // split K and the XCD-major tile numbering
  const int cuss[] = {256, 304, 80};
  const int toks[] = {1, 8, 16, 31, 32, 33, 64, 96, 127, 128, 129, 2048};
  const int64_t pks[] = {128, 1024, 4096, 8192, 14336, 16384, 28672, 131072};
  for (int cus : cuss)
    for (int T : toks)
      for (int64_t n : rows)
        for (int64_t k : pks) check_splitk(T, (int)n, (int)k, cus);
  // BitDelta: M <= 8192 (8 waves of 1024 codes), N up to the 2^31-byte base range
  const int64_t brow[] = {1, 7, 37, 100, 513, 8192, 65535, 131071, 1000000};
  for (int cap : {256, 512, 1024, 80})
    for (int64_t n : brow)
      for (int m : {16, 208, 1024, 1040, 4096, 8192}) {
        if (n * m * 2 >= (int64_t(1) << 31)) continue;
        check_bitdelta(n, m, cap);
      }
  printf("%s: %ld plans checked, %ld failed checks\n", g_fail ? "FAILED" : "ok", g_cases, g_fail);
  return g_fail ? 1 : 0;
}
