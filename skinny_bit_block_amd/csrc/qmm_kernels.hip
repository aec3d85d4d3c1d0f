// HIP kernels (gfx950) of the skinny quantized product
//   y[M,N] = x[M,K] . dequant(W)[N,K]^T,  M = 1..32,
// W in 144-byte / 256-weight Q4_K super-blocks (layout in include/qmm.h).
//
// The pages' finding ("sixi-asi 0.9", section "What I got wrong in 0.8") is
// that a kernel which decodes the 4-bit weights again for every row makes the
// verify pass pay per row. Here every super-block is loaded once and
// dequantized once, in registers, and that one decode serves all M rows.
//
// Work split, common to both kernels: a wavefront owns 16 consecutive rows n
// (a row tile). Lane l = 16 g + r handles row r of the tile and the j-pair g
// (sub-blocks 2g and 2g+1, i.e. weights 64g .. 64g+63 of each super-block):
// it loads the block header (16 B) and the 32 quant bytes 32g .. 32g+31 with
// 128-bit loads. Those bytes hold weights 64g+i (low nibble of byte i) and
// 64g+32+i (high nibble). A row tile walks the super-blocks of its K slice in
// ascending order; each workgroup first stages its K slice of x in LDS, rounded
// once to binary16 and arranged to match the nibble order, together with the
// fp32 sums of every 32-weight sub-block of the rounded x (the min term).
//
// Nibble unpack: masking a quant dword with 0x000F000F leaves two binary16
// subnormals q*2^-24 (bytes 0 and 2, low nibbles); 0x00F000F0 leaves q*2^-20
// (high nibbles); the same after a shift by 8 gives bytes 1 and 3. gfx950
// keeps binary16 subnormals in v_dot2_f32_f16, v_pk_mul_f16 and the f16 MFMA,
// so this is exact and needs no bias correction.
//
// Row-vector kernel (VALU): per row m, v_dot2_f32_f16 of the unpacked quants
// with the staged x, two fp32 partial sums per lane (one per sub-block), then
//   y += d*sc_a*2^24 * P_a + d*sc_b*2^20 * P_b - dmin*m_a*S_a - dmin*m_b*S_b.
// Tiled kernel (MFMA): the quants are scaled by their sub-block scale with one
// v_pk_mul_f16 per pair (q*sc*2^-14, exact: q*sc <= 945), the staged x is the
// A operand and the weights the B operand of v_mfma_f32_16x16x32_f16, so a
// lane's four outputs belong to its own row n and the per-block d is a lane
// constant; the min term is a v_mfma_f32_16x16x4_f32 of the sub-block sums
// with -dmin*m_j. Accumulation is fp32 in a fixed order in both kernels.
// With split-K, every slice writes its partial sums, and the wave that
// finishes a row tile last (an atomic arrival counter per tile) adds the
// partials in slice order and writes y, then resets the counter for the next
// call; which wave is last does not change the order of the sum, so results
// are bit-identical from run to run for a given launch plan, and a call is a
// single kernel launch. Each wave walks a fixed sequence of row tiles of one K
// slice (persistent workgroups).
//
// The tiled kernel has three more instantiations: the expert-indexed product
// (IDS: row m multiplies matrix ids[m]; "sixi-asi 0.9", section "The patch",
// names the MUL_MAT_ID op), block-scaled FP4 weights (FMT = 1: E2M1 codes
// with one E4M3 scale per 16, repacked by the host into the same 144-byte
// geometry, decoded with gfx950's packed FP4 conversion; FlashRT issue #153
// measures an NVFP4 W4A16 product, the format's bits are the OCP MX / OFP8
// specifications') and plain INT4 weights (FMT = 2: two's-complement codes
// with one binary16 scale per 128 columns, "sixi-asi 0.11", section "What
// did not work"; same geometry, exact code decode, two MFMA chains per group).
//
// x staging (both kernels): a workgroup loads all its x units at once (16 B of
// binary16 each, loaded in row order so eight lanes read one 128-byte run),
// issues its first weight stage, waits for x alone (s_waitcnt vmcnt with the
// stage still outstanding), converts, and stores in the kernel's LDS layout;
// the tiled layout XORs each unit's row slot with a function of its position
// so the stores spread over all LDS banks (x_lead, x_issue, x_finish below).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "qmm_internal.h"

namespace qmm {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), c,
                                false);
}

__device__ __forceinline__ uint32_t pk_mul(uint32_t a, h2_t s) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, a) * s);
}

__device__ __forceinline__ float f16_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Header of a super-block, the part lane group g needs: d, dmin and the
// scales/mins of sub-blocks 2g (a) and 2g+1 (b).
struct Header {
  float d, dmin;
  uint32_t sc_a, sc_b, m_a, m_b;
};

// Per-lane constants of the header decode. The twelve packed scale bytes are
// s0..s3 = h.y, s4..s7 = h.z, s8..s11 = h.w. Lane group g needs
//   g < 2:  sc = s[2g], s[2g+1] (low 6 bits), m = s[4+2g], s[5+2g] (low 6 bits)
//   g >= 2 (t = g-2): low 4 bits from s[8+2t], s[9+2t] (scale: low nibble,
//          min: high nibble), bits 4..5 from the top two bits of s[2t], s[2t+1]
//          (scale) and of s[4+2t], s[5+2t] (min).
// One v_perm_b32 gathers the four low-part bytes, one gathers the four
// high-part bytes, and per-lane masks finish the job: bytes [sc_a, sc_b, m_a, m_b].
struct HeaderLane {
  uint32_t sel_lo, mask_a, mask_b, sel_hi, mask_h;
  bool hi_group;
};

__device__ __forceinline__ HeaderLane header_lane(int g) {
  HeaderLane c;
  const uint32_t t = (uint32_t)(g & 1) * 2u;
  c.hi_group = g >= 2;
  if (g < 2) {
    c.sel_lo = t | ((t + 1) << 8) | ((4 + t) << 16) | ((5 + t) << 24);
    c.mask_a = 0x3F3F3F3Fu;
    c.mask_b = 0u;
    c.sel_hi = 0x0C0C0C0Cu;  // selector 12 = zero byte
    c.mask_h = 0u;
  } else {
    c.sel_lo = t | ((t + 1) << 8) | (t << 16) | ((t + 1) << 24);
    c.mask_a = 0x00000F0Fu;
    c.mask_b = 0x0F0F0000u;
    c.sel_hi = t | ((t + 1) << 8) | ((4 + t) << 16) | ((5 + t) << 24);
    c.mask_h = 0x30303030u;
  }
  return c;
}

// [sc_a, sc_b, m_a, m_b] as the four bytes of one dword.
__device__ __forceinline__ uint32_t scale_bytes(u4_t h, const HeaderLane& c) {
  const uint32_t s0 = c.hi_group ? h.w : h.z;
  const uint32_t s1 = c.hi_group ? h.w : h.y;
  uint32_t lo = __builtin_amdgcn_perm(s0, s1, c.sel_lo);
  lo = (lo & c.mask_a) | ((lo >> 4) & c.mask_b);
  const uint32_t hi = __builtin_amdgcn_perm(h.z, h.y, c.sel_hi);
  return ((hi >> 2) & c.mask_h) | lo;
}

__device__ __forceinline__ Header decode_header(u4_t h, const HeaderLane& c) {
  Header o;
  o.d = f16_lo(h.x);
  o.dmin = f16_hi(h.x);
  const uint32_t b = scale_bytes(h, c);
  o.sc_a = b & 0xFFu;
  o.sc_b = (b >> 8) & 0xFFu;
  o.m_a = (b >> 16) & 0xFFu;
  o.m_b = b >> 24;
  return o;
}

// Stage x[0..M)[K slice] into LDS: unit (m, bl, g, t) holds, as binary16
// pairs, x at block offsets 64g + {4t, 4t+2 | 4t+1, 4t+3 | 32+4t, 32+4t+2 |
// 32+4t+1, 32+4t+3}; sums[m][bl][j] is the fp32 sum of the rounded x over
// sub-block j. The eight lanes t = 0..7 of a (m, bl, g) group are adjacent,
// so the sub-block sums are a fixed xor-butterfly over those lanes.
// All x units of a workgroup are loaded at once when they fit in U units per
// thread (U = kVectorLead or kTiledLead); a larger slice first stages chunks
// of U units per thread one after another. The last chunk's loads are issued
// before the first weight stage, and its conversion waits only for them (an
// s_waitcnt that leaves the weight stage's kStageLoads loads outstanding), so
// x and the first weights are in flight together. Every load of a chunk is
// issued unconditionally (lanes past the end re-read the last unit), which
// keeps the compiler's wait counts exact.
constexpr int kVectorLead = 8;
constexpr int kTiledLead = 16;

template <int U>
struct XRegs {
  f4_t lo[U], hi[U];  // native vectors (HIP's float4 wrapper kept them out of registers)
};

struct StageArgs {
  const float* x;
  int M, K, kb0, nbw, xs_m, ss_m;
  int Mx;  // tiled kernel: row slots of the staged x (tiled_x_rows)
  char* lds_x;
  float* lds_s;
  int rowreg;  // with an expert map: lane k holds the x row of local row k
  bool remap;
};

// x row of local row m (the caller's own row unless rows are gathered)
__device__ __forceinline__ int x_row(const StageArgs& a, int m) {
  return a.remap ? __shfl(a.rowreg, m) : m;
}

// q = u / d for u < 2^24 and 1 <= d <= 32: a float estimate is within one of
// the quotient; one correction step makes it exact.
__device__ __forceinline__ int div_small(int u, int d, float rcp) {
  int q = (int)((float)u * rcp);
  const int rem = u - q * d;
  q += rem < 0 ? -1 : (rem >= d ? 1 : 0);
  return q;
}

// Sum over the 8 aligned lanes of a group, in every lane of it, with DPP
// (VALU, no LDS traffic; the compiler folds each move into a v_add_f32_dpp):
// quad_perm [1,0,3,2] and [2,3,0,1] leave the quad's sum in each lane (fp32
// addition is commutative, so all four agree), row_half_mirror then adds the
// other quad of the eight.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float sum8(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  return v;
}

// Two fp32 values rounded to binary16 (nearest-even) and packed, a in the
// low half: one v_cvt_pk_f16_f32.
typedef float f2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, h2_t));
}
// c + the two binary16 values of p, in fp32 (one v_dot2 with ones).
__device__ __forceinline__ float hsum2(uint32_t p, float c) {
  const h2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, p), ones, c, false);
}

// Unit order of the staging loads: u = ((bl*M + m)*4 + g)*8 + t, so the 8
// consecutive lanes t = 0..7 read one contiguous 128-byte run of a row (the
// kernels' LDS layouts are computed from (m, bl, g, t) when storing). A probe
// measured this order about 4x faster than reading in the tiled kernel's LDS
// order, where each load instruction touches 64 rows-and-segments.
// A thread's units of one chunk are base + j*nthr + threadIdx.x, j = 0, 1, ...
// Their t and g are the thread's own (nthr is a multiple of 32); (m, bl)
// advance by the quotient and remainder of nthr/32 by M at each step.
struct XWalk {
  int m, bl;
  int dq, dr;
};
__device__ __forceinline__ XWalk xwalk(int base, int M, float rcp) {
  const int rest = (base + (int)threadIdx.x) >> 5;
  const int bl = div_small(rest, M, rcp);
  const int s = (int)blockDim.x >> 5;
  const int dq = div_small(s, M, rcp);
  return XWalk{rest - bl * M, bl, dq, s - dq * M};
}
__device__ __forceinline__ void xstep(XWalk& w, int M) {
  w.m += w.dr;
  w.bl += w.dq;
  if (w.m >= M) {
    w.m -= M;
    ++w.bl;
  }
}

// Tiled x layout: unit (m, bl, g, t) of c-row c = (bl*8 + t)*4 + g sits in
// row slot m ^ xswz(t, g, Mx) of that c-row (Mx slots of 16 B). Without the
// swizzle the staging stores, whose 16-lane groups take t = 0..7 and two g of
// one row, all fall into the same LDS banks for Mx >= 16 (a probe: 64 cycles
// per store instead of 4.6); with it they cover 16 distinct 16-byte slots
// (Mx >= 8; 2-way at most below), while the MFMA reads of a c-row (16 rows at
// fixed t, g) remain a permutation of 16 slots (measured at the same cost).
__device__ __forceinline__ int xswz(int t, int g, int Mx) {
  return Mx >= 16 ? ((2 * t + (g & 1)) & 15) : (t & (Mx - 1));
}

// Loads of a chunk: nu units per thread. Lanes past the last unit re-read a
// unit of the slice (row M-1, last block) and store nothing.
template <int U>
__device__ __forceinline__ void x_issue(const StageArgs& a, int base, int nu, float rcp,
                                        XRegs<U>& b) {
  const int last = a.M * a.nbw * 32 - 1;
  const int nthr = (int)blockDim.x;
  const int t = (int)threadIdx.x & 7, g = ((int)threadIdx.x >> 3) & 3;
  const uint32_t c0 = (uint32_t)(a.kb0 * kBlockWeights + 64 * g + 4 * t);
  const uint32_t clamp = (uint32_t)x_row(a, a.M - 1) * (uint32_t)a.K +
                         (uint32_t)(a.nbw - 1) * kBlockWeights + c0;
  XWalk w = xwalk(base, a.M, rcp);
#pragma unroll
  for (int j = 0; j < U; ++j) {
    if (j < nu) {  // uniform across the workgroup
      const int u = base + j * nthr + (int)threadIdx.x;
      const uint32_t off =
          u <= last ? (uint32_t)x_row(a, w.m) * (uint32_t)a.K + (uint32_t)(w.bl << 8) + c0 : clamp;
      const float* src = a.x + off;
      b.lo[j] = *reinterpret_cast<const f4_t*>(src);
      b.hi[j] = *reinterpret_cast<const f4_t*>(src + 32);
      xstep(w, a.M);
    }
  }
}

// Layouts of the staged activations (units of 16 B = 8 binary16 values):
//   row-vector kernel: the 32 dwords d = 4t + c of (m, bl, g) at
//     m*xs_m + bl*512 + g*128, dword d at position 2*(d % 16) + d / 16, so
//     lane r of a 16-lane row reads dwords r and 16 + r with one 8-byte load;
//     sums[m][bl][j] at m*ss_m + bl*8 + j;
//   tiled kernel: unit (m, bl, g, t) at
//     16*(((bl*8 + t)*4 + g)*Mx + (m ^ xswz(t, g, Mx))), so the 16 lanes of a
//     j-pair read the units of one c-row (rows past M repeat real rows);
//     sums of (m, bl, g) as a float2 at 8*((bl*4 + g)*M + m).
// dwords of a unit: x at block offsets 64g + {4t, 4t+2 | 4t+1, 4t+3 |
// 32+4t, 32+4t+2 | 32+4t+1, 32+4t+3}, the order of the B operand's nibbles.
// The sub-block sums come from the same rounded values: a unit's four, then a
// DPP sum over the eight lanes t = 0..7 of its (m, bl, g) group, which are
// adjacent in the load order (every lane takes part; only valid units store).
// PAIRED (the FP4 instantiation of the tiled kernel): each dword holds x at
// block offsets (64g + 4t + i, 64g + 32 + 4t + i), i = 0..3, the pairs the
// hardware FP4 conversion produces from one code byte; no sub-block sums.
template <bool TILED, int U, bool PAIRED = false>
__device__ __forceinline__ void x_finish(const StageArgs& a, int base, int nu, float rcp,
                                         const XRegs<U>& b) {
  const int nunits = a.M * a.nbw * 32;
  const int nthr = (int)blockDim.x;
  const int t = (int)threadIdx.x & 7, g = ((int)threadIdx.x >> 3) & 3;
  const int sw = xswz(t, g, a.Mx);
  const int cslot = (4 * t + g) * a.Mx;
  const int lgblk = 5 + (31 - __builtin_clz(a.Mx));  // slots per super-block: 32 * Mx
  const int p0 = t < 4 ? 8 * t : 8 * (t - 4) + 1;  // row-vector: position of dword 4t
  XWalk w = xwalk(base, a.M, rcp);
#pragma unroll
  for (int j = 0; j < U; ++j) {
    if (j < nu) {  // uniform
      const int u = base + j * nthr + (int)threadIdx.x;
      u4_t v;
      float slo = 0.f, shi = 0.f;
      if (PAIRED) {
        v.x = cvt_pk(b.lo[j][0], b.hi[j][0]);
        v.y = cvt_pk(b.lo[j][1], b.hi[j][1]);
        v.z = cvt_pk(b.lo[j][2], b.hi[j][2]);
        v.w = cvt_pk(b.lo[j][3], b.hi[j][3]);
      } else {
        v.x = cvt_pk(b.lo[j][0], b.lo[j][2]);
        v.y = cvt_pk(b.lo[j][1], b.lo[j][3]);
        v.z = cvt_pk(b.hi[j][0], b.hi[j][2]);
        v.w = cvt_pk(b.hi[j][1], b.hi[j][3]);
        slo = sum8(hsum2(v.x, hsum2(v.y, 0.f)));
        shi = sum8(hsum2(v.z, hsum2(v.w, 0.f)));
      }
      if (u < nunits) {
        if (TILED) {
          const int slot = (w.bl << lgblk) + cslot + (w.m ^ sw);
          *reinterpret_cast<u4_t*>(a.lds_x + 16 * slot) = v;
          if (!PAIRED && t == 0)
            *reinterpret_cast<float2*>(a.lds_s + 2 * ((w.bl * 4 + g) * a.M + w.m)) =
                float2{slo, shi};
        } else {
          uint32_t* dst = reinterpret_cast<uint32_t*>(a.lds_x + w.m * a.xs_m + w.bl * 512 + g * 128);
          dst[p0] = v.x;
          dst[p0 + 2] = v.y;
          dst[p0 + 4] = v.z;
          dst[p0 + 6] = v.w;
          if (t == 0) {
            a.lds_s[w.m * a.ss_m + w.bl * 8 + 2 * g] = slo;
            a.lds_s[w.m * a.ss_m + w.bl * 8 + 2 * g + 1] = shi;
          }
        }
      }
      xstep(w, a.M);
    }
  }
}

// Stages every chunk but the last and issues the last one's loads; returns
// that chunk's first unit and sets nu to its units per thread.
template <bool TILED, int U, bool PAIRED = false>
__device__ __forceinline__ int x_lead(const StageArgs& a, float rcp, XRegs<U>& b, int& nu) {
  const int nthr = (int)blockDim.x;
  int left = (a.M * a.nbw * 32 + nthr - 1) / nthr;
  int base = 0;
  for (; left > U; left -= U, base += U * nthr) {
    x_issue<U>(a, base, U, rcp, b);
    x_finish<TILED, U, PAIRED>(a, base, U, rcp, b);
  }
  x_issue<U>(a, base, left, rcp, b);
  nu = left;
  return base;
}

// Wait until at most n vector-memory operations of this wave are outstanding
// (gfx9 encoding: vmcnt in bits 3:0, expcnt and lgkmcnt at their maxima, so
// only vmcnt is waited for).
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | n);
}

struct Quants {
  uint32_t a[8], e[8], b[8], f[8];  // see the file comment: a,e low nibbles; b,f high
};

__device__ __forceinline__ void unpack(const u4_t& q0, const u4_t& q1, Quants& o) {
  const uint32_t d[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t s = d[t] >> 8;
    o.a[t] = d[t] & 0x000F000Fu;
    o.b[t] = d[t] & 0x00F000F0u;
    o.e[t] = s & 0x000F000Fu;
    o.f[t] = s & 0x00F000F0u;
  }
}

__device__ __forceinline__ u4_t load_nt(const u4_t* p) { return __builtin_nontemporal_load(p); }

// Weight stream. A wavefront reads its 16 rows in stages of kStageBlocks
// super-blocks: the stage is 16 row segments of 576 contiguous bytes, read by
// kStageLoads 128-bit loads per lane in which consecutive lanes take
// consecutive 16-byte chunks (chunk q = lane + 64 i is row q / 36, chunk
// q % 36 of that row's segment). Every load instruction thus covers about two
// long contiguous runs instead of sixteen scattered pieces, which is what lets
// the memory system run near its streaming rate. The chunks go through a
// wave-private LDS buffer (row stride 37 chunks, so the compute reads below
// hit distinct banks) from which lane (r, g) reads its block header and its
// 32 quant bytes. While a stage is being computed the next one is in flight.
constexpr int kStageBlocks = 4;
constexpr int kSegChunks = 9 * kStageBlocks;          // 36 chunks of 16 B per row
constexpr int kStageLoads = 16 * kSegChunks / 64;     // 9 loads per lane
constexpr int kBufRowStride = 16 * (kSegChunks + 1);  // 592 B

struct StageRegs {
  u4_t v[kStageLoads];
};

// Per-lane constants of the stage loads: byte offset of chunk i inside the
// wave's slice (row and position) and its LDS address. Row tiles differ only
// in their base address, except a last tile with fewer than 16 rows, whose
// missing rows re-read its last row (those lanes are never stored).
struct StageLane {
  uint32_t goff[kStageLoads];  // row * (nb * 144) + chunk * 16, stage 0
  uint32_t loff[kStageLoads];  // LDS byte offset from the dynamic LDS base
  int blk[kStageLoads];        // super-block of the chunk within a stage
};

__device__ __forceinline__ void stage_lane(int lane, int nb, int rows, uint32_t wbuf,
                                           StageLane& c) {
#pragma unroll
  for (int i = 0; i < kStageLoads; ++i) {
    const int q = lane + 64 * i;
    const int row = q / kSegChunks, cc = q % kSegChunks;
    const int rr = min(row, rows - 1);
    c.blk[i] = cc / 9;
    c.goff[i] = (uint32_t)(rr * nb * kBlockBytes + cc * 16);  // a block is 9 chunks
    c.loff[i] = wbuf + (uint32_t)(row * kBufRowStride + cc * 16);
  }
}

// Issue the loads of stage s (super-blocks 4s .. 4s+3 of the slice). A full
// stage is a wave-uniform base plus each lane's 32-bit offsets (no vector
// address arithmetic); in a partial last stage, chunks past the slice end
// re-read the slice's last block and are never used.
__device__ __forceinline__ void stage_load(const uint8_t* wave_base, const StageLane& c, int s,
                                           int nbw, StageRegs& sr) {
  const uint8_t* sbase = wave_base + (size_t)s * (kStageBlocks * kBlockBytes);
  if ((s + 1) * kStageBlocks <= nbw) {
#pragma unroll
    for (int i = 0; i < kStageLoads; ++i)
      sr.v[i] = load_nt(reinterpret_cast<const u4_t*>(sbase + c.goff[i]));
  } else {
    const int last = nbw - 1 - s * kStageBlocks;  // last valid block of this stage
#pragma unroll
    for (int i = 0; i < kStageLoads; ++i) {
      const uint32_t back = c.blk[i] > last ? (uint32_t)((c.blk[i] - last) * kBlockBytes) : 0u;
      sr.v[i] = load_nt(reinterpret_cast<const u4_t*>(sbase + (c.goff[i] - back)));
    }
  }
}

__device__ __forceinline__ void stage_store(char* lds, const StageLane& c, const StageRegs& sr) {
#pragma unroll
  for (int i = 0; i < kStageLoads; ++i) *reinterpret_cast<u4_t*>(lds + c.loff[i]) = sr.v[i];
}

// The first stage of a wave's first tile. A wave without one (no tile, or no
// K work) loads a stage of the matrix's first rows instead, which it never
// stores: every wave then has exactly kStageLoads loads outstanding after its
// x loads, the count the prologue's s_waitcnt relies on.
__device__ __forceinline__ void first_stage(const uint8_t* W, const uint8_t* slice_base, int tile,
                                            int ntiles, int nstages, int nb, int N, int nbw,
                                            size_t row_bytes, int lane, uint32_t wbuf,
                                            StageLane& sl, StageRegs& sr) {
  const bool real = tile < ntiles && nstages > 0;
  const int t = real ? tile : 0;
  stage_lane(lane, nb, min(16, N - t * 16), wbuf, sl);
  stage_load(real ? slice_base + (size_t)t * 16 * row_bytes : W, sl, 0, real ? nbw : nb, sr);
}

// One super-block as lane (r, g) needs it: the header and its j-pair's quants.
struct BlockRegs {
  u4_t hd, qa, qb;
};

__device__ __forceinline__ void read_block(const char* rowbuf, int g, int j, BlockRegs& b) {
  const char* base = rowbuf + 9 * j * 16;
  b.hd = *reinterpret_cast<const u4_t*>(base);
  b.qa = *reinterpret_cast<const u4_t*>(base + 16 + 32 * g);
  b.qb = *reinterpret_cast<const u4_t*>(base + 32 + 32 * g);
}

// Split-K. Partials are agent-scope atomic stores (performed at the device's
// coherence point); once they are complete (s_waitcnt) one relaxed atomic add
// on the tile's counter announces them. The wave that sees splits-1 reads the
// other slices with agent-scope atomic loads, sums all slices in slice order,
// and resets the counter. No L2 write-back or invalidate is needed because
// every access to the partials is an agent-scope atomic.
__device__ __forceinline__ void store_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_partial(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool arrive_last(unsigned* counter, int splits, int lane) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  unsigned old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (old != (unsigned)(splits - 1)) return false;
  if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Sum of all slices of one output in slice order; the caller's own slice comes
// from its register (bitwise the value it stored).
__device__ __forceinline__ float sum_slices(const float* ws, size_t mn, int splits, int own,
                                            float own_v, size_t idx) {
  float v = own == 0 ? own_v : load_partial(ws + idx);
  for (int k = 1; k < splits; ++k) v += (k == own) ? own_v : load_partial(ws + (size_t)k * mn + idx);
  return v;
}

// Work split inside a workgroup. Its waves form T = waves / wsplit tile groups
// of wsplit waves; the waves of a group reduce consecutive K slices of the same
// row tile, and their partial sums meet in LDS (in slice order, after a
// barrier) instead of in global memory. The workgroups of one slice range walk
// the row tiles round-robin; every wave of a workgroup runs the same number of
// tile iterations, so the barrier is uniform.
struct Split {
  int wslice, wtile, T;  // this wave's slice within the workgroup, its tile group, groups
  int kb0, nbw;          // this wave's K slice: first super-block, count (may be 0)
  int bl_off;            // its first super-block within the workgroup's staged x
  int kb0_wg, nbw_wg;    // the workgroup's K range
  int iters;             // tile iterations of the workgroup
};

__device__ __forceinline__ Split make_split(int wave, int waves, int wsplit, int nbs, int nb,
                                            int ntiles) {
  Split c;
  c.wslice = wave % wsplit;
  c.wtile = wave / wsplit;
  c.T = waves / wsplit;
  c.kb0_wg = (int)blockIdx.y * wsplit * nbs;
  c.nbw_wg = min(wsplit * nbs, nb - c.kb0_wg);
  c.bl_off = c.wslice * nbs;
  c.kb0 = c.kb0_wg + c.bl_off;
  c.nbw = max(0, min(nbs, nb - c.kb0));
  const int first_wg = (int)blockIdx.x * c.T;
  const int step = (int)gridDim.x * c.T;
  c.iters = first_wg < ntiles ? (ntiles - 1 - first_wg) / step + 1 : 0;
  return c;
}

// LDS buffer of the in-workgroup reduction: floats [parity][tile group][slice][m][16],
// parity = iteration & 1 (one barrier per iteration then suffices).
__device__ __forceinline__ float* red_slot(float* red, int par, const Split& c, int wsplit,
                                           int slice, int M) {
  return red + (size_t)(((par * c.T + c.wtile) * wsplit + slice) * M) * 16;
}

// Output of one row tile: NV values per lane, for output rows grow[k] (ok[k]:
// the row exists) of output column n. Writes y, or with split-K across
// workgroups the partial and, for the last slice to arrive, the sum of all
// slices in slice order. Mtot rows of y, counter ctr of the tile.
template <int NV>
__device__ __forceinline__ void write_tile(const float (&v)[NV], const int (&grow)[NV],
                                           const bool (&ok)[NV], int n, int N, int Mtot, int ctr,
                                           float* __restrict__ y, float* __restrict__ ws,
                                           unsigned* __restrict__ counters, int lane) {
  const int gsplits = (int)gridDim.y, gslice = (int)blockIdx.y;
  if (gsplits == 1) {
    if (n < N) {
#pragma unroll
      for (int k = 0; k < NV; ++k)
        if (ok[k]) y[(size_t)grow[k] * N + n] = v[k];
    }
    return;
  }
  const size_t mn = (size_t)Mtot * (size_t)N;
  if (n < N) {
#pragma unroll
    for (int k = 0; k < NV; ++k)
      if (ok[k]) store_partial(ws + (size_t)gslice * mn + (size_t)grow[k] * N + n, v[k]);
  }
  if (arrive_last(counters + ctr, gsplits, lane) && n < N) {
#pragma unroll
    for (int k = 0; k < NV; ++k)
      if (ok[k])
        y[(size_t)grow[k] * N + n] =
            sum_slices(ws, mn, gsplits, gslice, v[k], (size_t)grow[k] * N + n);
  }
}

// One tile iteration's end: with wsplit > 1 the slices' partials meet in LDS
// (indexed by local row mrow) and the tile group's first wave writes the tile.
// Every wave of the workgroup calls this once per iteration (it contains the
// barrier).
template <int NV>
__device__ __forceinline__ void finish_tile(float (&v)[NV], const int (&mrow)[NV],
                                            const int (&grow)[NV], const bool (&ok)[NV],
                                            bool valid, int it, const Split& c, int wsplit,
                                            float* red, int r, int n, int N, int M, int Mtot,
                                            int ctr, float* __restrict__ y,
                                            float* __restrict__ ws, unsigned* __restrict__ counters,
                                            int lane) {
  if (wsplit == 1) {
    if (valid) write_tile<NV>(v, grow, ok, n, N, Mtot, ctr, y, ws, counters, lane);
    return;
  }
  const int par = it & 1;
  if (valid) {
    float* mine = red_slot(red, par, c, wsplit, c.wslice, M);
#pragma unroll
    for (int k = 0; k < NV; ++k)
      if (ok[k]) mine[mrow[k] * 16 + r] = v[k];
  }
  __syncthreads();
  if (valid && c.wslice == 0) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (!ok[k]) continue;
      float sum = v[k];  // slice 0 is this wave's own
      for (int sl = 1; sl < wsplit; ++sl) sum += red_slot(red, par, c, wsplit, sl, M)[mrow[k] * 16 + r];
      v[k] = sum;
    }
    write_tile<NV>(v, grow, ok, n, N, Mtot, ctr, y, ws, counters, lane);
  }
}

// ---------------------------------------------------------------- row-vector
// Eight v_dot2c_f32_f16 whose first operand is an x dword broadcast from lane
// n of the lane's 16-lane row (DPP row_newbcast:n): lanes of a row share their
// j-pair, so each holds two of its 32 x dwords and the row reads them from one
// another without touching LDS. The compiler cannot see hazards inside asm, so
// the asm keeps two distances itself. A DPP instruction must not read a VGPR
// that a VALU instruction wrote in the two previous slots, so every block of
// eight starts with s_nop 1 for the operands written just before it. And the
// tied accumulator of a DPP dot is read back later than that: on gfx950 a dot
// that reads its accumulator four slots after the previous dot wrote it adds
// to a stale value, so the eight dots of a block write eight different
// accumulators, and each is read again seven dots later at the earliest.
#define QMM_DOT(acc, w, n) "v_dot2c_f32_f16_dpp %[" acc "], %[x], %[" w "] row_newbcast:" #n " row_mask:0xf bank_mask:0xf\n"
#define QMM_DOT8(n0, n1, n2, n3, n4, n5, n6, n7)                                            \
  "s_nop 1\n" QMM_DOT("c0", "w0", n0) QMM_DOT("c1", "w1", n1) QMM_DOT("c2", "w2", n2)        \
      QMM_DOT("c3", "w3", n3) QMM_DOT("c4", "w4", n4) QMM_DOT("c5", "w5", n5)              \
          QMM_DOT("c6", "w6", n6) QMM_DOT("c7", "w7", n7)
#define QMM_DOT_OPERANDS(T)                                                                    \
  : [c0] "+v"(p.c[0]), [c1] "+v"(p.c[1]), [c2] "+v"(p.c[2]), [c3] "+v"(p.c[3]),                \
    [c4] "+v"(p.c[4]), [c5] "+v"(p.c[5]), [c6] "+v"(p.c[6]), [c7] "+v"(p.c[7])                 \
  : [x] "v"(x), [w0] "v"(q.a[T]), [w1] "v"(q.e[T]), [w2] "v"(q.b[T]), [w3] "v"(q.f[T]),       \
    [w4] "v"(q.a[T + 1]), [w5] "v"(q.e[T + 1]), [w6] "v"(q.b[T + 1]), [w7] "v"(q.f[T + 1])

// c0, c1, c4, c5 sum low nibbles (sub-block 2g), c2, c3, c6, c7 high nibbles
// (sub-block 2g+1)
struct DotAcc {
  float c[8];
};

// dwords d = 4t + c of the j-pair for t = T, T+1: c = 0, 1 feed P_a (low
// nibbles, sub-block 2g), c = 2, 3 feed P_b (high nibbles, sub-block 2g+1)
template <int T>
__device__ __forceinline__ void dots8(DotAcc& p, uint32_t x, const Quants& q) {
  if (T % 4 == 0)
    asm(QMM_DOT8(0, 1, 2, 3, 4, 5, 6, 7) QMM_DOT_OPERANDS(T));
  else
    asm(QMM_DOT8(8, 9, 10, 11, 12, 13, 14, 15) QMM_DOT_OPERANDS(T));
}

template <int M>
__device__ __forceinline__ void vector_block(const BlockRegs& br, const HeaderLane& hl,
                                             const char* xl, const float* sg, int bl, int xs_m,
                                             int ss_m, float (&acc)[M]) {
  const Header h = decode_header(br.hd, hl);
  const float ca = h.d * (float)h.sc_a * 16777216.0f;  // 2^24: undo the low-nibble scale
  const float cb = h.d * (float)h.sc_b * 1048576.0f;   // 2^20: undo the high-nibble scale
  const float ma = -h.dmin * (float)h.m_a;
  const float mb = -h.dmin * (float)h.m_b;
  Quants q;
  unpack(br.qa, br.qb, q);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    // this lane's two x dwords of (m, block, j-pair): d = r and d = 16 + r
    const uint2 xv = *reinterpret_cast<const uint2*>(xl + m * xs_m + bl * 512);
    DotAcc p{{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}};
    dots8<0>(p, xv.x, q);
    dots8<2>(p, xv.x, q);
    dots8<4>(p, xv.y, q);
    dots8<6>(p, xv.y, q);
    const float pa = (p.c[0] + p.c[1]) + (p.c[4] + p.c[5]);
    const float pb = (p.c[2] + p.c[3]) + (p.c[6] + p.c[7]);
    const float2 s = *reinterpret_cast<const float2*>(sg + m * ss_m + bl * 8);
    float v = acc[m];
    v = fmaf(ca, pa, v);
    v = fmaf(cb, pb, v);
    v = fmaf(ma, s.x, v);
    v = fmaf(mb, s.y, v);
    acc[m] = v;
  }
}

// Issue order at kernel start: every wave first issues its share of the x
// loads, then the workgroup passes a barrier, and only then are weight loads
// issued; so the small x reads, which every workgroup needs before it can
// compute, are not queued behind a whole stage of weight streams.
__device__ __forceinline__ void issue_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int M>
__global__ void __launch_bounds__(512) qmm_vector_kernel(const float* __restrict__ x,
                                                         const uint8_t* __restrict__ W,
                                                         float* __restrict__ y,
                                                         float* __restrict__ ws,
                                                         unsigned* __restrict__ counters, int N,
                                                         int K, int nbs, int wsplit, int xs_m,
                                                         int ss_m) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int nb = K / kBlockWeights;
  const int waves = (int)blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // uniform per wave
  const int lane = (int)threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int ntiles = (N + 15) >> 4;
  const Split c = make_split(wave, waves, wsplit, nbs, nb, ntiles);
  const int tile_step = (int)gridDim.x * c.T;
  const int nstages = (c.nbw + kStageBlocks - 1) / kStageBlocks;
  const size_t row_bytes = (size_t)nb * kBlockBytes;
  const uint8_t* slice_base = W + (size_t)c.kb0 * kBlockBytes;

  char* lds_x = lds;
  float* lds_s = reinterpret_cast<float*>(lds + M * xs_m);
  const int red_base = lds_red_base(M, M, xs_m, ss_m);
  float* red = reinterpret_cast<float*>(lds + red_base);
  const uint32_t wbuf =
      (uint32_t)(red_base + lds_red_bytes(M, waves, wsplit) + wave * 16 * kBufRowStride);
  const StageArgs st{x, M, K, c.kb0_wg, c.nbw_wg, xs_m, ss_m, M, lds_x, lds_s, 0, false};
  XRegs<kVectorLead> xb;
  int xnu;
  const float rcp = 1.0f / (float)M;
  const int xbase = x_lead<false, kVectorLead>(st, rcp, xb, xnu);
  issue_barrier();
  int tile = (int)blockIdx.x * c.T + c.wtile;
  StageLane sl;
  StageRegs sr;
  first_stage(W, slice_base, tile, ntiles, nstages, nb, N, c.nbw, row_bytes, lane, wbuf, sl, sr);
  wait_vm<kStageLoads>();  // x complete; the first weight stage stays in flight
  x_finish<false, kVectorLead>(st, xbase, xnu, rcp, xb);
  __syncthreads();

  const HeaderLane hl = header_lane(g);
  const char* xl = lds_x + g * 128 + 8 * r;
  const float* sg = lds_s + 2 * g;
  const char* rowbuf = lds + wbuf + r * kBufRowStride;
  constexpr int NV = (M + 3) / 4;  // rows m = g + 4k of this lane's outputs
  int mrow[NV];
  bool ok[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    mrow[k] = min(g + 4 * k, M - 1);
    ok[k] = g + 4 * k < M;
  }
  // one flat loop over (tile, stage) steps with a single load site; a wave
  // without K work takes one empty step per tile, so every wave reaches
  // finish_tile (and its barrier) once per tile iteration
  const int ns = max(nstages, 1);
  const int total = c.iters * ns;
  int cs = 0, it = 0;
  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.f;
  for (int e = 0; e < total; ++e) {
    const bool valid = tile < ntiles;
    if (valid && nstages > 0) {
      stage_store(lds, sl, sr);
      int nt = tile, nsn = cs + 1;
      if (nsn == nstages) {
        nsn = 0;
        nt += tile_step;
      }
      if (nt < ntiles) {
        if (nsn == 0 && N - nt * 16 < 16) stage_lane(lane, nb, N - nt * 16, wbuf, sl);
        stage_load(slice_base + (size_t)nt * 16 * row_bytes, sl, nsn, c.nbw, sr);
      }
      const int bl0 = cs * kStageBlocks;
      if (bl0 + kStageBlocks <= c.nbw) {
        // full stage: one basic block, so the scheduler can overlap blocks
#pragma unroll
        for (int j = 0; j < kStageBlocks; ++j) {
          BlockRegs br;
          read_block(rowbuf, g, j, br);
          vector_block<M>(br, hl, xl, sg, c.bl_off + bl0 + j, xs_m, ss_m, acc);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kStageBlocks; ++j) {
          if (bl0 + j < c.nbw) {
            BlockRegs br;
            read_block(rowbuf, g, j, br);
            vector_block<M>(br, hl, xl, sg, c.bl_off + bl0 + j, xs_m, ss_m, acc);
          }
        }
      }
    }
    if (++cs == ns) {
      // the four lanes of a row (g = 0..3) hold its four j-pair partials
      float v[NV];
#pragma unroll
      for (int k = 0; k < NV; ++k) v[k] = 0.f;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float t = acc[m];
        t += __shfl_xor(t, 16);
        t += __shfl_xor(t, 32);
        if ((m & 3) == g) v[m >> 2] = t;
        acc[m] = 0.f;
      }
      finish_tile<NV>(v, mrow, mrow, ok, valid, it, c, wsplit, red, r, tile * 16 + r, N, M, M,
                      tile, y, ws, counters, lane);
      cs = 0;
      ++it;
      tile += tile_step;
    }
  }
}

// --------------------------------------------------------------------- tiled
// The tiled kernel's activations are staged by x_lead / x_finish
// above: unit (m, bl, g, t) at LDS byte 16*(((bl*8 + t)*4 + g)*M + m).

template <int MT>
__device__ __forceinline__ void tiled_block(const BlockRegs& br, const HeaderLane& hl,
                                            const char* lds_x, const int (&xo)[MT][8],
                                            const float* const (&sa)[MT], int bl, int M, int Mx,
                                            f4_t (&acc)[MT]) {
  const Header h = decode_header(br.hd, hl);
  const _Float16 sa16 = (_Float16)(float)(h.sc_a * 1024u);  // q*2^-24 -> q*sc*2^-14
  const _Float16 sb16 = (_Float16)(float)(h.sc_b * 64u);    // q*2^-20 -> q*sc*2^-14
  const h2_t sca = {sa16, sa16}, scb = {sb16, sb16};
  const float dd = h.d * 16384.0f;  // 2^14
  const float ma = -h.dmin * (float)h.m_a;
  const float mb = -h.dmin * (float)h.m_b;
  Quants q;
  unpack(br.qa, br.qb, q);
  h8_t bw[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    u4_t v;
    v.x = pk_mul(q.a[t], sca);
    v.y = pk_mul(q.e[t], sca);
    v.z = pk_mul(q.b[t], scb);
    v.w = pk_mul(q.f[t], scb);
    bw[t] = __builtin_bit_cast(h8_t, v);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const char* xp = lds_x + bl * 512 * Mx;
    f4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 8; ++t)
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          __builtin_bit_cast(h8_t, *reinterpret_cast<const u4_t*>(xp + xo[mt][t])), bw[t], c, 0,
          0, 0);
    f4_t a = acc[mt];
    a[0] = fmaf(dd, c[0], a[0]);
    a[1] = fmaf(dd, c[1], a[1]);
    a[2] = fmaf(dd, c[2], a[2]);
    a[3] = fmaf(dd, c[3], a[3]);
    const float2 s = *reinterpret_cast<const float2*>(sa[mt] + bl * 8 * M);
    a = __builtin_amdgcn_mfma_f32_16x16x4f32(s.x, ma, a, 0, 0, 0);
    a = __builtin_amdgcn_mfma_f32_16x16x4f32(s.y, mb, a, 0, 0, 0);
    acc[mt] = a;
  }
}

// Block-scaled FP4 groups (qmm_run_nvfp4): 256 weights in 144 bytes like the
// 4.5-bit super-blocks, bytes 0..15 the E4M3 scale codes of the 16 runs of 16
// weights, bytes 16..143 the E2M1 element codes in the same byte and nibble
// order as the 4-bit quants. Lane (r, g) reads its j-pair's four scale codes
// (runs 4g..4g+3) with one 4-byte load and its 32 code bytes as before.
__device__ __forceinline__ void read_block_fp4(const char* rowbuf, int g, int j, BlockRegs& b) {
  const char* base = rowbuf + 9 * j * 16;
  b.hd.x = *reinterpret_cast<const uint32_t*>(base + 4 * g);
  b.qa = *reinterpret_cast<const u4_t*>(base + 16 + 32 * g);
  b.qb = *reinterpret_cast<const u4_t*>(base + 32 + 32 * g);
}

// Two E4M3 codes (bytes 0 and 2 of p) to a binary16 pair, exactly: placing a
// code's exponent and mantissa bits at binary16 bits 13..7 and its sign at bit
// 15 gives its value x 2^-8 (normal and subnormal codes alike, as both formats
// have the same structure below the exponent bias), and x 256 is exact.
__device__ __forceinline__ h2_t e4m3_pair(uint32_t p) {
  const uint32_t v = ((p & 0x007F007Fu) << 7) | ((p & 0x00800080u) << 8);
  const h2_t k = {(_Float16)256.0f, (_Float16)256.0f};
  return __builtin_bit_cast(h2_t, v) * k;
}

// One group for the lane's 16 rows. v_cvt_scalef32_pk_f16_fp4 turns code
// byte i of dword t into the binary16 pair (weight 64g + 4t + i, weight
// 64g + 32 + 4t + i), exactly (scale 1; a probe on the MI355X matched all 256
// bytes at every byte position against the E2M1 table), and one v_pk_mul_f16
// applies the pair's two scales (runs 4g + t/4 and 4g + 2 + t/4). The x of
// this instantiation is staged in the same pairs (x_finish PAIRED). A product
// of a code and a scale is exact in binary16: (8+m)*n*2^(E-4) with
// (8+m)*n <= 180 and E >= -6, or k*n*2^-10 for subnormal scales. So the MFMAs
// accumulate straight into the tile and the tensor scale is applied once per
// output (oscale = the tensor scale).
template <int MT>
__device__ __forceinline__ void tiled_block_fp4(const BlockRegs& br, const char* lds_x,
                                                const int (&xo)[MT][8], int bl, int Mx,
                                                f4_t (&acc)[MT]) {
  const uint32_t sc = br.hd.x;  // codes of runs 4g, 4g+1, 4g+2, 4g+3
  const h2_t sa = e4m3_pair(__builtin_amdgcn_perm(0u, sc, 0x0C020C00u));  // (4g, 4g+2)
  const h2_t sb = e4m3_pair(__builtin_amdgcn_perm(0u, sc, 0x0C030C01u));  // (4g+1, 4g+3)
  const uint32_t d[8] = {br.qa.x, br.qa.y, br.qa.z, br.qa.w, br.qb.x, br.qb.y, br.qb.z, br.qb.w};
  h8_t bw[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const h2_t s2 = t < 4 ? sa : sb;
    u4_t v;
    v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d[t], 1.0f, 0) * s2);
    v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d[t], 1.0f, 1) * s2);
    v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d[t], 1.0f, 2) * s2);
    v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d[t], 1.0f, 3) * s2);
    bw[t] = __builtin_bit_cast(h8_t, v);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const char* xp = lds_x + bl * 512 * Mx;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          __builtin_bit_cast(h8_t, *reinterpret_cast<const u4_t*>(xp + xo[mt][t])), bw[t],
          acc[mt], 0, 0, 0);
  }
}

// Plain 4-bit integer groups (qmm_run_int4): 256 weights in 144 bytes like the
// 4.5-bit super-blocks, bytes 0..3 the binary16 scales of weights 0..127 and
// 128..255, bytes 16..143 the codes in the same byte and nibble order as the
// 4-bit quants, stored offset by 8 (u = q + 8). The masks of unpack leave u as
// binary16 subnormals u*2^-24 (low nibbles) and u*2^-20 (high nibbles); one
// packed add (or fma with 1/16) of -8*2^-24 turns each pair into q*2^-24
// exactly, so zero codes give exact zeros. Lane (r, g)'s j-pair lies in scale
// group g/2, and an MFMA spans all four j-pairs, so each block runs two MFMA
// chains: chain c reads x (A) only in the lanes of group c and a zero chunk of
// LDS in the others (xa/xb: per-lane offsets and block strides), and the two
// results are scaled by the row's two scales in fp32.
template <int MT>
__device__ __forceinline__ void tiled_block_int4(const BlockRegs& br, const char* lds,
                                                 const uint32_t (&xa)[2][MT][8],
                                                 const uint32_t (&xb)[2], int bl,
                                                 f4_t (&acc)[MT]) {
  const float s0 = f16_lo(br.hd.x) * 16777216.0f;  // 2^24: undo the code scaling
  const float s1 = f16_hi(br.hd.x) * 16777216.0f;
  Quants q;
  unpack(br.qa, br.qb, q);
  const h2_t m8 = {(_Float16)-0x1p-21f, (_Float16)-0x1p-21f};  // -8 * 2^-24
  const h2_t r16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  h8_t bw[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    u4_t v;
    v.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, q.a[t]) + m8);
    v.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, q.e[t]) + m8);
    v.z = __builtin_bit_cast(uint32_t,
                             __builtin_elementwise_fma(__builtin_bit_cast(h2_t, q.b[t]), r16, m8));
    v.w = __builtin_bit_cast(uint32_t,
                             __builtin_elementwise_fma(__builtin_bit_cast(h2_t, q.f[t]), r16, m8));
    bw[t] = __builtin_bit_cast(h8_t, v);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    f4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
    const uint32_t b0 = (uint32_t)bl * xb[0], b1 = (uint32_t)bl * xb[1];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const u4_t a0 = *reinterpret_cast<const u4_t*>(lds + b0 + xa[0][mt][t]);
      const u4_t a1 = *reinterpret_cast<const u4_t*>(lds + b1 + xa[1][mt][t]);
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a0), bw[t], c0, 0, 0,
                                                  0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a1), bw[t], c1, 0, 0,
                                                  0);
    }
    f4_t a = acc[mt];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = fmaf(s1, c1[i], fmaf(s0, c0[i], a[i]));
    acc[mt] = a;
  }
}

// Expert-indexed calls (ids != nullptr): row m multiplies expert ids[m] of E
// consecutive matrices (expert_bytes apart). grid.z enumerates the distinct
// experts in ascending order; the workgroups of slot z stream that expert's
// matrix once for all rows that use it (M of them, gathered through a lane
// register map) and scatter the results. Rows whose id is outside [0, E) are
// not written. Without ids, slot 0 is the whole call.
struct Slot {
  int M;           // rows of this slot
  int rowreg;      // lane k: the caller's row of local row k
  bool remap;
  const uint8_t* W;
  int ctr_base;    // first split-K counter of this slot
  bool empty;      // no expert for this slot
};

__device__ __forceinline__ Slot make_slot(const int* __restrict__ ids, int E, long long expert_bytes,
                                          const uint8_t* W, int Mtot, int ntiles, int lane) {
  Slot o{Mtot, lane, false, W, 0, false};
  if (!ids) return o;
  const int id = lane < Mtot ? ids[lane] : -1;
  const bool valid = id >= 0 && id < E;
  bool first = valid;  // no earlier row has the same id
  for (int j = 0; j < Mtot; ++j) {
    const int oj = __shfl(id, j);
    if (j < lane && oj == id) first = false;
  }
  const unsigned long long fmask = __ballot(first);
  int rank = 0;  // distinct valid ids below this one
  for (int j = 0; j < Mtot; ++j) {
    const int oj = __shfl(id, j);
    if (((fmask >> j) & 1ull) && oj < id) ++rank;
  }
  const unsigned long long pick = __ballot(first && rank == (int)blockIdx.z);
  if (pick == 0ull) {
    o.empty = true;
    return o;
  }
  const int e = __shfl(id, (int)__builtin_ctzll(pick));
  const unsigned long long match = __ballot(valid && id == e);
  o.M = (int)__popcll(match);
  for (int j = 0; j < Mtot; ++j)
    if (((match >> j) & 1ull) && (int)__popcll(match & ((1ull << j) - 1ull)) == lane) o.rowreg = j;
  o.remap = true;
  o.W = W + (size_t)e * (size_t)expert_bytes;
  o.ctr_base = (int)blockIdx.z * ntiles;
  return o;
}

// FMT 0: 4.5-bit k-quant super-blocks; FMT 1: block-scaled FP4 groups, whose
// outputs are multiplied by oscale (the tensor scale).
template <int MT, bool IDS, int FMT>
__global__ void __launch_bounds__(512) qmm_tiled_kernel(const float* __restrict__ x,
                                                        const uint8_t* __restrict__ W,
                                                        float* __restrict__ y,
                                                        float* __restrict__ ws,
                                                        unsigned* __restrict__ counters, int Mtot,
                                                        int N, int K, int nbs, int wsplit,
                                                        int xs_m, int ss_m,
                                                        const int* __restrict__ ids, int E,
                                                        long long expert_bytes, float oscale) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int nb = K / kBlockWeights;
  const int waves = (int)blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // uniform per wave
  const int lane = (int)threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int ntiles = (N + 15) >> 4;
  const Slot sl0 = IDS ? make_slot(ids, E, expert_bytes, W, Mtot, ntiles, lane)
                       : Slot{Mtot, lane, false, W, 0, false};
  if (IDS && sl0.empty) return;  // the same for every wave of the workgroup
  const int M = sl0.M;    // rows of this call (or of this expert)
  const Split c = make_split(wave, waves, wsplit, nbs, nb, ntiles);
  const int tile_step = (int)gridDim.x * c.T;
  const int nstages = (c.nbw + kStageBlocks - 1) / kStageBlocks;
  const size_t row_bytes = (size_t)nb * kBlockBytes;
  const uint8_t* slice_base = sl0.W + (size_t)c.kb0 * kBlockBytes;

  // LDS regions are laid out for Mtot rows; this slot uses the first M
  const int Mx = tiled_x_rows(Mtot);
  char* lds_x = lds;
  float* lds_s = reinterpret_cast<float*>(lds + Mx * xs_m);
  const int red_base = lds_red_base(Mx, Mtot, xs_m, ss_m);
  float* red = reinterpret_cast<float*>(lds + red_base);
  const uint32_t wbuf =
      (uint32_t)(red_base + lds_red_bytes(Mtot, waves, wsplit) + wave * 16 * kBufRowStride);
  const StageArgs st{x, M, K, c.kb0_wg, c.nbw_wg, xs_m, ss_m, Mx, lds_x, lds_s, sl0.rowreg, IDS};
  const float rcp = 1.0f / (float)M;
  XRegs<kTiledLead> xb;
  int xnu;
  const int xbase = x_lead<true, kTiledLead, FMT == 1>(st, rcp, xb, xnu);
  issue_barrier();
  int tile = (int)blockIdx.x * c.T + c.wtile;
  StageLane sl;
  StageRegs sr;
  first_stage(sl0.W, slice_base, tile, ntiles, nstages, nb, N, c.nbw, row_bytes, lane, wbuf, sl,
              sr);
  wait_vm<kStageLoads>();  // x complete; the first weight stage stays in flight
  x_finish<true, kTiledLead, FMT == 1>(st, xbase, xnu, rcp, xb);
  // INT4: a zero 16-byte chunk after the wave buffers (the A operand of the
  // lanes outside a chain's scale group)
  const uint32_t zoff = (uint32_t)(red_base + lds_red_bytes(Mtot, waves, wsplit) +
                                   waves * kWaveBufBytes);
  if (FMT == 2 && threadIdx.x == 0) *reinterpret_cast<u4_t*>(lds + zoff) = u4_t{0u, 0u, 0u, 0u};
  __syncthreads();

  const HeaderLane hl = header_lane(g);
  // A-operand row this lane reads in each 16-row MFMA tile. An MFMA output row
  // depends only on its A row and rows past M are never stored, so padded
  // rows re-read a real row of the same tile. xo: the row's unit of c-row
  // 4t + g within a super-block (swizzled slot), per tile and t.
  int xo[MT][8];
  const float* sa[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int rows = min(M - 16 * mt, 16);
    const int m = 16 * mt + r % rows;
#pragma unroll
    for (int t = 0; t < 8; ++t) xo[mt][t] = 16 * ((4 * t + g) * Mx + (m ^ xswz(t, g, Mx)));
    sa[mt] = lds_s + 2 * (g * M + m);
  }
  // INT4: chain c's A operand is x in the lanes of scale group c (j-pairs 2c,
  // 2c+1) and the zero chunk elsewhere: offset xa + bl * xb
  uint32_t xa[2][MT][8], xbs[2];
  if (FMT == 2) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bool own = (g >> 1) == c;
      xbs[c] = own ? (uint32_t)(512 * Mx) : 0u;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 8; ++t) xa[c][mt][t] = own ? (uint32_t)xo[mt][t] : zoff;
    }
  }
  const char* rowbuf = lds + wbuf + r * kBufRowStride;
  constexpr int NV = 4 * MT;  // rows m = 16 mt + 4 g + i of this lane's outputs
  int mrow[NV], grow[NV];
  bool ok[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int m = 16 * (k >> 2) + 4 * g + (k & 3);
    mrow[k] = min(m, M - 1);
    ok[k] = m < M;
    grow[k] = IDS ? __shfl(sl0.rowreg, mrow[k]) : mrow[k];
  }
  const int ns = max(nstages, 1);
  const int total = c.iters * ns;
  int cs = 0, it = 0;
  f4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f4_t{0.f, 0.f, 0.f, 0.f};
  for (int e = 0; e < total; ++e) {
    const bool valid = tile < ntiles;
    if (valid && nstages > 0) {
      stage_store(lds, sl, sr);
      int nt = tile, nsn = cs + 1;
      if (nsn == nstages) {
        nsn = 0;
        nt += tile_step;
      }
      if (nt < ntiles) {
        if (nsn == 0 && N - nt * 16 < 16) stage_lane(lane, nb, N - nt * 16, wbuf, sl);
        stage_load(slice_base + (size_t)nt * 16 * row_bytes, sl, nsn, c.nbw, sr);
      }
      const int bl0 = cs * kStageBlocks;
      if (bl0 + kStageBlocks <= c.nbw) {
        // full stage: one basic block, so the scheduler can overlap blocks
#pragma unroll
        for (int j = 0; j < kStageBlocks; ++j) {
          BlockRegs br;
          if (FMT == 1) {
            read_block_fp4(rowbuf, g, j, br);
            tiled_block_fp4<MT>(br, lds_x, xo, c.bl_off + bl0 + j, Mx, acc);
          } else if (FMT == 2) {
            read_block(rowbuf, g, j, br);
            tiled_block_int4<MT>(br, lds, xa, xbs, c.bl_off + bl0 + j, acc);
          } else {
            read_block(rowbuf, g, j, br);
            tiled_block<MT>(br, hl, lds_x, xo, sa, c.bl_off + bl0 + j, M, Mx, acc);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < kStageBlocks; ++j) {
          if (bl0 + j < c.nbw) {
            BlockRegs br;
            if (FMT == 1) {
              read_block_fp4(rowbuf, g, j, br);
              tiled_block_fp4<MT>(br, lds_x, xo, c.bl_off + bl0 + j, Mx, acc);
            } else if (FMT == 2) {
              read_block(rowbuf, g, j, br);
              tiled_block_int4<MT>(br, lds, xa, xbs, c.bl_off + bl0 + j, acc);
            } else {
              read_block(rowbuf, g, j, br);
              tiled_block<MT>(br, hl, lds_x, xo, sa, c.bl_off + bl0 + j, M, Mx, acc);
            }
          }
        }
      }
    }
    if (++cs == ns) {
      float v[NV];
#pragma unroll
      for (int k = 0; k < NV; ++k) v[k] = FMT == 1 ? acc[k >> 2][k & 3] * oscale : acc[k >> 2][k & 3];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f4_t{0.f, 0.f, 0.f, 0.f};
      finish_tile<NV>(v, mrow, grow, ok, valid, it, c, wsplit, red, r, tile * 16 + r, N, M, Mtot,
                      sl0.ctr_base + tile, y, ws, counters, lane);
      cs = 0;
      ++it;
      tile += tile_step;
    }
  }
}

// Entry points: [rows - 1] for the row-vector kernel (1..8 rows: its VALU
// work grows with every row, and the tiled kernel is faster from 2 rows),
// [MFMA row tiles - 1] for the tiled kernel.
#define QMM_V(m) reinterpret_cast<const void*>(&qmm_vector_kernel<m>)
const void* const kVectorFn[kMaxVectorRows] = {QMM_V(1), QMM_V(2), QMM_V(3), QMM_V(4),
                                               QMM_V(5), QMM_V(6), QMM_V(7), QMM_V(8)};
#undef QMM_V
// [plain, expert-indexed, block-scaled FP4, plain INT4][row tiles - 1]
const void* const kTiledFn[4][2] = {
    {reinterpret_cast<const void*>(&qmm_tiled_kernel<1, false, 0>),
     reinterpret_cast<const void*>(&qmm_tiled_kernel<2, false, 0>)},
    {reinterpret_cast<const void*>(&qmm_tiled_kernel<1, true, 0>),
     reinterpret_cast<const void*>(&qmm_tiled_kernel<2, true, 0>)},
    {reinterpret_cast<const void*>(&qmm_tiled_kernel<1, false, 1>),
     reinterpret_cast<const void*>(&qmm_tiled_kernel<2, false, 1>)},
    {reinterpret_cast<const void*>(&qmm_tiled_kernel<1, false, 2>),
     reinterpret_cast<const void*>(&qmm_tiled_kernel<2, false, 2>)}};

const void* kernel_fn(int kernel, int M) {
  if (M < 1 || M > 32) return nullptr;
  if (kernel == 1) return M <= kMaxVectorRows ? kVectorFn[M - 1] : nullptr;
  if (kernel >= 2 && kernel <= 5) return kTiledFn[kernel - 2][M > 16 ? 1 : 0];
  return nullptr;
}

// Scratch of the entry point that allocates nothing (qmm_run_static): the
// split-K partial sums, then one 32-bit arrival counter per row tile, in one
// file-scope device array. Every device the library runs on holds its own
// copy until the process ends. Host code never passes the array's name to a
// kernel (on the host it only stands for the symbol): static_scratch()
// resolves the device address once per device and every launch uses that.
static __device__ __align__(256) unsigned char scratch[kStaticPartialBytes + kStaticCounterTiles * 4];

__global__ void zero_u32(unsigned* __restrict__ p, int n) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = 0u;
}

constexpr int kMaxStaticDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxStaticDevices];

}  // namespace

hipError_t static_scratch(int device, void** out) {
  if (device < 0 || device >= kMaxStaticDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));  // current device
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

hipError_t clear_counters(unsigned* counters, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_u32, dim3((n + 255) / 256), dim3(256), 0, stream, counters, n);
  return hipGetLastError();
}

hipError_t prepare_kernels() {
  for (int m = 0; m < kMaxVectorRows; ++m) {
    hipError_t e = hipFuncSetAttribute(kVectorFn[m], hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
    if (e != hipSuccess) return e;
  }
  for (int t = 0; t < 8; ++t) {
    hipError_t e = hipFuncSetAttribute(kTiledFn[t >> 1][t & 1],
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t resident_per_cu(int kernel, int M, int waves, int lds_bytes, int* out) {
  const void* f = kernel_fn(kernel, M);
  if (!f) return hipErrorInvalidValue;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, f, 64 * waves, (size_t)lds_bytes);
}

hipError_t launch(const Launch& a, hipStream_t stream) {
  const void* f = kernel_fn(a.kernel, a.M);
  if (!f) return hipErrorInvalidValue;
  const dim3 grid(a.grid_x, a.grid_y, a.slots), block(64 * a.waves_per_wg);
  const uint8_t* W = static_cast<const uint8_t*>(a.W);
  int M = a.M, N = a.N, K = a.K, nbs = a.nbs, wsplit = a.wsplit, xs_m = a.xs_m, ss_m = a.ss_m;
  const float* x = a.x;
  float* y = a.y;
  float* ws = a.ws;
  unsigned* counters = a.counters;
  const int* ids = a.ids;
  int E = a.E;
  long long expert_bytes = a.expert_bytes;
  float oscale = a.oscale;
  if (a.kernel != 1) {
    void* args[] = {&x, &W, &y, &ws, &counters, &M, &N, &K, &nbs, &wsplit, &xs_m, &ss_m,
                    &ids, &E, &expert_bytes, &oscale};
    if (a.ev_start || a.ev_stop)
      return hipExtLaunchKernel(f, grid, block, args, (size_t)a.lds_bytes, stream, a.ev_start,
                                a.ev_stop, 0);
    return hipLaunchKernel(f, grid, block, args, (size_t)a.lds_bytes, stream);
  }
  void* args[] = {&x, &W, &y, &ws, &counters, &N, &K, &nbs, &wsplit, &xs_m, &ss_m};
  if (a.ev_start || a.ev_stop)
    return hipExtLaunchKernel(f, grid, block, args, (size_t)a.lds_bytes, stream, a.ev_start,
                              a.ev_stop, 0);
  return hipLaunchKernel(f, grid, block, args, (size_t)a.lds_bytes, stream);
}

}  // namespace qmm
