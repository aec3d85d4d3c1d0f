// Gated DeltaNet recurrent update with the replay of a row log
// (include/gdn.h): one base state per sequence, the kept rows of its log and
// its new rows applied in one kernel ("sixi-asi 0.11", section "A log instead
// of snapshots"); the update is the gated delta rule of the Gated DeltaNet
// paper (Yang, Kautz and Hatamizadeh, ICLR 2025).
//
// Work split. Row i of a head's state evolves on its own given the row's
// inputs: s <- alpha s + beta (v_i - alpha (s . k)) k, o_i = s . q. One
// workgroup takes one head of one sequence with 8 waves: the two halves of
// the 128 value rows (a lane per value row) times the four quarters of the
// 128 key indices. A lane keeps its 32 state values in VGPRs for the whole
// walk (the state is read once and written at most once per call, which is
// the HBM traffic of the step), and the quarters' partial dot products meet
// in LDS once per row. Keys, queries, gates and betas are the same for every
// lane of a wave: uniform loads through the scalar cache whose values are
// SGPR operands of the per-element FMAs. The state layout [B][H][dk][dv]
// puts a wave's 64 value rows of one key index in one contiguous 256-byte run,
// so every state load and store is coalesced. Small per-lane state leaves
// room for many waves per SIMD, which is what hides the latency of the row
// loop (the scalar loads of each row's vectors, the exchange). The state and
// the outputs are each touched once per call, so their loads and stores are
// non-temporal (they do not displace the rows' inputs, which every wave of a
// head reads, from the caches).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn.h"
#include "../../include/qmm.h"

namespace {

constexpr int kDk = 128;
constexpr int kDv = 128;
constexpr int kHalves = 2;                 // value-row halves of a head (64 lanes each)
constexpr int kQuarters = 4;               // key-index quarters
constexpr int kKq = kDk / kQuarters;       // 32 state values per lane
constexpr int kThreads = kDv * kQuarters;  // 512 threads: 8 waves

// The inputs every lane of a wave reads alike (keys, queries, gates, betas)
// are read through the constant address space: the call never writes them
// (the host checks that no input overlaps the state or o), and loads from it
// become scalar loads whatever the walk stores to o and to the state (through
// a global pointer the compiler cannot prove that after the commit's stores
// and falls back to vector loads of the uniform data).
typedef __attribute__((address_space(4))) const float cfloat;

// Inputs of one call as one wave walks them.
struct Walk {
  cfloat* k_log;
  const float* __restrict__ v_log;
  cfloat* g_log;
  cfloat* b_log;
  cfloat* q;
  cfloat* k;
  const float* __restrict__ v;
  cfloat* g;
  cfloat* beta;
  float* __restrict__ o;
  int b, h, H, M, L, nl, T, i, e0;  // e0: this wave's first key index
};

// Row r of the walk: a kept row of the log (r < nl) or new row r - nl.
struct RowRef {
  cfloat* k;  // this wave's quarter of the key
  float vi, alpha, beta;
  bool fresh;
  size_t row;  // index of the row's (b, row, h) entries
};

__device__ __forceinline__ size_t row_index(const Walk& w, int r) {
  return r >= w.nl ? ((size_t)w.b * w.M + (r - w.nl)) * w.H + w.h
                   : ((size_t)w.b * w.L + r) * w.H + w.h;
}

__device__ __forceinline__ RowRef row_ref(const Walk& w, int r) {
  RowRef x;
  x.fresh = r >= w.nl;
  x.row = row_index(w, r);
  x.k = (x.fresh ? w.k : w.k_log) + x.row * kDk + w.e0;
  x.vi = (x.fresh ? w.v : w.v_log)[x.row * kDv + w.i];
  x.alpha = (x.fresh ? w.g : w.g_log)[x.row];
  x.beta = (x.fresh ? w.beta : w.b_log)[x.row];
  return x;
}

// z . kr over the lane's 32 values, in four interleaved partial sums (a fixed
// order: calls are bitwise repeatable)
__device__ __forceinline__ float dot32(const float (&z)[kKq], cfloat* kr) {
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
  for (int e = 0; e < kKq; e += 4) {
    a0 = __builtin_fmaf(z[e], kr[e], a0);
    a1 = __builtin_fmaf(z[e + 1], kr[e + 1], a1);
    a2 = __builtin_fmaf(z[e + 2], kr[e + 2], a2);
    a3 = __builtin_fmaf(z[e + 3], kr[e + 3], a3);
  }
  return (a0 + a1) + (a2 + a3);
}

// The lane keeps its state values as s = P * z: P the product of the gates
// applied since the last fold (the same in every wave of the workgroup) and z
// in registers. A row then changes z by one FMA per element,
// z <- z + (u / P') k with P' = alpha P (the decay is the scalar P' instead
// of a multiply per element), and s . w = P (z . w). z is folded (z <- P z,
// P <- 1) after any row that takes P below 2^-64, which a scan of the gates
// finds before the rows run, and P' is kept at or above 2^-100: a gate small
// enough to hit that floor decays the old state by 2^-100 instead of less,
// a relative error of at most 2^-36 (the fold came at most 2^64 earlier).
// Everything else is the row's update rounded in binary32, so the error
// allowance per row is that of the plain update.
constexpr float kFold = 0x1.0p-64f;
constexpr float kFloor = 0x1.0p-100f;

// The scaled gate product after a row, kept at or above the floor.
__device__ __forceinline__ float next_scale(float P, float alpha) {
  return __builtin_fmaxf(P * alpha, kFloor);
}

// Per-row exchange of the quarters' partial sums through LDS: slot
// [parity][quarter][value row] holds (s . k of the next row, s . q of this
// row), each already scaled by P. Two parities: a wave may write row r + 1's
// slot while another still reads row r's; the barrier of row r + 1 orders
// the reuse of row r's slot.
struct Exchange {
  float2 (*slot)[kQuarters][kDv];
  int par;
};

// Publish this wave's partials, wait for the workgroup, and sum the four
// quarters in quarter order (the same order in every wave, so every wave of
// a half gets the same a and o).
__device__ __forceinline__ float2 exchange(Exchange& x, const Walk& w, int quarter, float2 part) {
  x.slot[x.par][quarter][w.i] = part;
  __syncthreads();
  float2 t = x.slot[x.par][0][w.i];
#pragma unroll
  for (int qq = 1; qq < kQuarters; ++qq) {
    const float2 p = x.slot[x.par][qq][w.i];
    t.x += p.x;
    t.y += p.y;
  }
  x.par ^= 1;
  return t;
}

// Rows [r0, r1) of the walk, all of them kept rows of the log (OUT = false)
// or all new rows (OUT = true, each followed by its output). Each row: the
// exchange that completes s . k_r (and the previous new row's output), then
// one pass over the lane's z: the update, the dot of the new z with the next
// row's key quarter and, for a new row, with q_r's quarter.
template <bool OUT>
__device__ __forceinline__ void walk_rows(const Walk& w, Exchange& x, int quarter,
                                          float (&z)[kKq], float& P, RowRef& cur, float2& part,
                                          size_t& out_row, int r0, int r1) {
  for (int r = r0; r < r1; ++r) {
    const float2 t = exchange(x, w, quarter, part);
    if (out_row != ~(size_t)0 && quarter == 0) __builtin_nontemporal_store(t.y, w.o + out_row * kDv + w.i);
    out_row = OUT ? cur.row : ~(size_t)0;
    const float u = cur.beta * (cur.vi - cur.alpha * t.x);  // t.x = s . k_r
    const float Pn = next_scale(P, cur.alpha);
    const float coef = u / Pn;
    // the next row's key (the last row dots with its own key; the result is unused)
    const RowRef nxt = row_ref(w, r + 1 < w.T ? r + 1 : r);
    cfloat* kr = cur.k;
    cfloat* kn = nxt.k;
    cfloat* qr = w.q + (OUT ? cur.row * kDk + w.e0 : 0);
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
    for (int e = 0; e < kKq; e += 4) {
      z[e] = __builtin_fmaf(coef, kr[e], z[e]);
      z[e + 1] = __builtin_fmaf(coef, kr[e + 1], z[e + 1]);
      z[e + 2] = __builtin_fmaf(coef, kr[e + 2], z[e + 2]);
      z[e + 3] = __builtin_fmaf(coef, kr[e + 3], z[e + 3]);
      if (OUT) {
        o0 = __builtin_fmaf(z[e], qr[e], o0);
        o1 = __builtin_fmaf(z[e + 1], qr[e + 1], o1);
        o2 = __builtin_fmaf(z[e + 2], qr[e + 2], o2);
        o3 = __builtin_fmaf(z[e + 3], qr[e + 3], o3);
      }
      a0 = __builtin_fmaf(z[e], kn[e], a0);
      a1 = __builtin_fmaf(z[e + 1], kn[e + 1], a1);
      a2 = __builtin_fmaf(z[e + 2], kn[e + 2], a2);
      a3 = __builtin_fmaf(z[e + 3], kn[e + 3], a3);
    }
    part.x = Pn * ((a0 + a1) + (a2 + a3));
    part.y = OUT ? Pn * ((o0 + o1) + (o2 + o3)) : 0.f;
    P = Pn;
    cur = nxt;
  }
}

// The first row after r at which the walk must fold z: the row after the
// first one that takes the scaled gate product (P at row r) below 2^-64, or
// `stop`. The same products as the walk's, so the walk's P after that row is
// below 2^-64 too.
__device__ __forceinline__ int fold_point(const Walk& w, int r, int stop, float P) {
  float p = P;
  for (int e = r; e < stop; ++e) {
    p = next_scale(p, (e >= w.nl ? w.g : w.g_log)[row_index(w, e)]);
    if (p < kFold) return e + 1;
  }
  return stop;
}

// One workgroup = one head of one sequence (blockIdx.x = b * H + h); wave
// 2 * quarter + half holds value rows [64 half, 64 half + 64) and key indices
// [32 quarter, 32 quarter + 32).
__global__ void __launch_bounds__(kThreads) gdn_replay_kernel(
    float* __restrict__ state, const float* __restrict__ k_log, const float* __restrict__ v_log,
    const float* __restrict__ g_log, const float* __restrict__ b_log,
    const int32_t* __restrict__ n_log, int L, const float* __restrict__ q,
    const float* __restrict__ k, const float* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, const int32_t* __restrict__ commit, float* __restrict__ o,
    int M, int H) {
  __shared__ float2 xch[2][kQuarters][kDv];
  const int bh = (int)blockIdx.x;
  const int h = bh % H, b = bh / H;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int half = wave % kHalves, quarter = wave / kHalves;
  const int i = half * 64 + ((int)threadIdx.x & 63);  // this lane's value row
  const int e0 = quarter * kKq;

  // the head's state (a wave-uniform base) and this lane's 32-bit offset
  float* const head = state + (size_t)bh * kDk * kDv;
  float z[kKq];
#pragma unroll
  for (int e = 0; e < kKq; ++e) z[e] = __builtin_nontemporal_load(head + (e0 + e) * kDv + i);
  float P = 1.f;

  int nl = n_log ? n_log[b] : 0;
  nl = nl < 0 ? 0 : (nl > L ? L : nl);
  const int T = nl + M;
  int c = commit ? commit[b] : 0;
  c = c < 0 ? 0 : (c > T ? T : c);
  if (T == 0) return;  // the whole workgroup

  const Walk w{(cfloat*)k_log, v_log, (cfloat*)g_log, (cfloat*)b_log, (cfloat*)q, (cfloat*)k, v,
               (cfloat*)g, (cfloat*)beta, o, b, h, H, M, L, nl, T, i, e0};
  Exchange x{xch, 0};
  RowRef cur = row_ref(w, 0);
  float2 part = make_float2(dot32(z, cur.k), 0.f);  // P = 1
  size_t out_row = ~(size_t)0;                      // a new row whose output is pending
  // segments of the walk end at the commit point, at fold points and at T;
  // every wave takes the same segments (they depend on the gates only)
  for (int r = 0; r < T;) {
    const int end = fold_point(w, r, r < c ? c : T, P);
    walk_rows<false>(w, x, quarter, z, P, cur, part, out_row, r, end < nl ? end : nl);
    walk_rows<true>(w, x, quarter, z, P, cur, part, out_row, r > nl ? r : nl, end);
    r = end;
    if (P < kFold) {  // fold (the pending partials are already scaled)
#pragma unroll
      for (int e = 0; e < kKq; ++e) z[e] *= P;
      P = 1.f;
    }
    if (r == c) {
      // the commit's store takes an opaque copy of the lane offset: its
      // addresses are formed here, not kept live from the loads at the top
      int li = i;
      asm("" : "+v"(li));
#pragma unroll
      for (int e = 0; e < kKq; ++e) __builtin_nontemporal_store(P * z[e], head + (e0 + e) * kDv + li);
    }
  }
  // the last new row's output
  if (out_row != ~(size_t)0) {
    const float2 t = exchange(x, w, quarter, part);
    if (quarter == 0) __builtin_nontemporal_store(t.y, o + out_row * kDv + i);
  }
}

bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + nb && pb < pa + na;
}

}  // namespace

extern "C" {

int gdn_replay_update(float* state, const float* k_log, const float* v_log,
                      const float* gate_log, const float* beta_log, const int32_t* n_log,
                      int64_t L, const float* q, const float* k, const float* v,
                      const float* gate, const float* beta, const int32_t* commit, float* o,
                      int64_t B, int64_t M, int64_t H, int64_t dk, int64_t dv,
                      hipStream_t stream) {
  if (!state || B < 1 || H < 1 || M < 0 || L < 0) return QMM_ERR_INVALID_ARG;
  if (dk != kDk || dv != kDv) return QMM_ERR_SHAPE;
  if (L > 0 && (!k_log || !v_log || !gate_log || !beta_log || !n_log)) return QMM_ERR_INVALID_ARG;
  if (M > 0 && (!q || !k || !v || !gate || !beta || !o)) return QMM_ERR_INVALID_ARG;
  if (B > INT32_MAX / H || L > INT32_MAX || M > INT32_MAX) return QMM_ERR_INVALID_ARG;
  // at most 2^40 rows of either kind, so that every byte count below is exact
  if ((uint64_t)(B * H) * (uint64_t)L > (1ull << 40) || (uint64_t)(B * H) * (uint64_t)M > (1ull << 40))
    return QMM_ERR_INVALID_ARG;
  const int64_t wgs = B * H;
  const void* ptrs[] = {state, k_log, v_log, gate_log, beta_log, n_log, q, k, v, gate, beta, commit, o};
  for (const void* p : ptrs)
    if ((uintptr_t)p & 3) return QMM_ERR_ALIGN;
  const uint64_t f = 4;
  const uint64_t sb = (uint64_t)B * H * kDk * kDv * f;
  const uint64_t lrow = (uint64_t)B * L * H, nrow = (uint64_t)B * M * H;
  struct Arr {
    const void* p;
    uint64_t n;
  };
  const Arr ins[] = {{k_log, lrow * kDk * f}, {v_log, lrow * kDv * f}, {gate_log, lrow * f},
                     {beta_log, lrow * f},    {n_log, L > 0 ? (uint64_t)B * 4 : 0},
                     {q, nrow * kDk * f},     {k, nrow * kDk * f},   {v, nrow * kDv * f},
                     {gate, nrow * f},        {beta, nrow * f},      {commit, commit ? (uint64_t)B * 4 : 0}};
  const uint64_t ob = nrow * kDv * f;
  if (overlaps(state, sb, o, ob)) return QMM_ERR_OVERLAP;
  for (const Arr& a : ins)
    if (overlaps(state, sb, a.p, a.n) || overlaps(o, ob, a.p, a.n)) return QMM_ERR_OVERLAP;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QMM_ERR_NO_DEVICE;
  hipLaunchKernelGGL(gdn_replay_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, stream, state,
                     k_log, v_log, gate_log, beta_log, L > 0 ? n_log : nullptr, (int)L, q, k, v,
                     gate, beta, commit, o, (int)M, (int)H);
  return hipGetLastError() == hipSuccess ? QMM_OK : QMM_ERR_HIP;
}

uint64_t gdn_call_bytes(int64_t B, int64_t M, int64_t H, int64_t dk, int64_t dv,
                        int64_t log_rows, int64_t committing) {
  if (B < 0 || M < 0 || H < 0 || dk < 0 || dv < 0 || log_rows < 0 || committing < 0) return 0;
  const uint64_t f = 4, head = (uint64_t)dk * dv * f;
  const uint64_t states = (uint64_t)B * H * head + (uint64_t)committing * H * head;
  const uint64_t logs = (uint64_t)log_rows * H * (dk + dv + 2) * f;
  const uint64_t fresh = (uint64_t)B * M * H * (2 * dk + dv + 2) * f;
  const uint64_t outs = (uint64_t)B * M * H * dv * f;
  return states + logs + fresh + outs;
}

}  // extern "C"
