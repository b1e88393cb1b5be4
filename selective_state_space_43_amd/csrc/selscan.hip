// libselscan -- selective state-space scan for AMD Instinct MI355X (gfx950).
//
// The operation (see include/selscan.h for the ABI):
//   delta_t = softplus(raw_t + bias),  Abar_t = exp(delta_t A),
//   h_t = Abar_t h_{t-1} + Bbar_t u_t,  y_t = (C_t . h_t + D u_t) silu(z_t)
// ("State-space models", sections "Discretization", "Recurrence and
// convolution", "Mamba: selection", "The parallel scan").
//
// Forward-scan design (gfx950, wave64):
//  * Lanes run along time.  A group of LPC lanes owns one channel (b, d); each
//    lane owns K consecutive timesteps of a chunk of LPC*K timesteps.  A wave
//    holds 64/LPC channels; a workgroup of W waves holds channels of one
//    sequence b, so the selective B_t, C_t (shared by every channel of a
//    sequence) are staged once per chunk in LDS as float32 and read by all
//    of them.
//  * Per state n each lane discretizes its K steps (one exp2 each), folds them
//    into one pair (prod Abar, local state) with the composition
//    (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2) ("Structured State Space Models
//    and Mamba ...", section "Hardware-Aware Parallel Associative Scan"),
//    the LPC lane pairs are scanned with DPP row shifts/broadcasts, the
//    channel's carry from the previous chunk is applied, and each lane
//    replays its K steps from its exact incoming state, accumulating the
//    readout C_t . h_t.  The expanded state never leaves registers.
//  * The chunk carry lives in LDS ([channels of the block][dstate]), so dstate
//    is a runtime value.  Step size, softplus, D skip and silu gate are fused.
//  * With 16 states, bf16 rows and many channels a second forward kernel runs
//    the recurrence in time order inside each lane instead (no fold, scan or
//    replay): lanes hold channels and states, the four waves of a workgroup
//    hold consecutive time segments and hand their states on through LDS
//    (scan_fwd_pipe_kernel below).
//  * Everything is float32; bf16 inputs are widened exactly, y is rounded to
//    bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32).
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <mutex>
#include <type_traits>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "selscan.h"

// Build-time tuning knobs of the forward scan (defaults are the tuned values).
#ifndef SELSCAN_K
#define SELSCAN_K 16  // timesteps per lane
#endif
#ifndef SELSCAN_W
#define SELSCAN_W 4  // waves per workgroup
#endif
#ifndef SELSCAN_NT
#define SELSCAN_NT 16  // states staged per LDS tile (16 lanes per channel)
#endif
#ifndef SELSCAN_PIPE_MIN_CHANNELS
// launches with 16 states and at least this many channels use the
// time-pipelined forward (one workgroup of four waves per 16 channels)
#define SELSCAN_PIPE_MIN_CHANNELS 8192
#endif
#ifndef SELSCAN_WAVES_PER_EU
// occupancy the register allocator must keep with 16 lanes per channel, for
// every rule and io type (0: no constraint): 3 waves per SIMD fit in 168
// VGPRs with some spills, and against 2 waves the bf16 forward runs about
// 1 % faster for delta*B, 11 % for exact ZOH, 15 % bilinear, 29 % Euler, and
// the float32 one 7-21 % faster (it spills more).  The wider lane layouts
// are held to two waves per SIMD by their grid and LDS: no constraint
#define SELSCAN_WAVES_PER_EU 3
#endif


namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- math

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = log(1 + e^x).  Above 15 it equals x to within 2e-8 relative.
// Below, log1p(e) is log(1 + e) with the rounding of 1 + e compensated to
// first order, which keeps relative accuracy for tiny e.
__device__ __forceinline__ float softplus_f(float x) {
  const float e = ex2(x * kLog2e);
  const float u = 1.0f + e;
  const float l = lg2(u) * kLn2 - ((u - 1.0f) - e) * rcp(u);
  return x > 15.0f ? x : l;
}

// softplus(x) / ln 2, the step size in log2 units, with the same accuracy.
// The rounding error of u = 1 + e is corrected to first order with 1/u
// replaced by 2 - u, which is exact enough wherever the correction matters
// (u near 1) and negligible where it does not.
__device__ __forceinline__ float softplus_log2(float x) {
  const float xl = x * kLog2e;
  const float e = ex2(xl);
  const float u = 1.0f + e;
  const float l = fmaf(((u - 1.0f) - e) * kLog2e, u - 2.0f, lg2(u));
  return x > 15.0f ? xl : l;
}

// softplus(raw + bias) / ln 2 from xl = (raw + bias) / ln 2 (formed by the
// caller as one fma), with the compensation of softplus_log2 and its factor
// (u - 2) / ln 2 as one fma.
__device__ __forceinline__ float softplus_xl(float xl) {
  const float e = ex2(xl);
  const float u = 1.0f + e;
  const float l = fmaf((u - 1.0f) - e, fmaf(u, kLog2e, -2.0f * kLog2e), lg2(u));
  return xl > 15.0f * kLog2e ? xl : l;
}

// silu(z) ln 2: the ln 2 goes into the reciprocal's argument for free.
__device__ __forceinline__ float silu_ln2(float z) {
  return z * rcp(fmaf(ex2(-z * kLog2e), kLog2e, kLog2e));
}


// silu(z) = z * sigmoid(z)
__device__ __forceinline__ float silu_f(float z) { return z * rcp(1.0f + ex2(-z * kLog2e)); }

// The exact zero-order-hold input coefficient (exp(delta A) - 1) / A from
// r = delta A, e = exp(r) and rA = 1 / A (0 when A = 0): (e - 1) rA, or, for
// |r| < 1/32 where e - 1 would cancel, delta (1 + r/2 + r^2/6 + r^3/24), whose
// first omitted term is below 1e-8 of the value; A = 0 gives delta.
__device__ __forceinline__ float zoh_coef(float r, float delta, float e, float rA) {
  const float p = delta * fmaf(r, fmaf(r, fmaf(r, 1.0f / 24, 1.0f / 6), 0.5f), 1.0f);
  return fabsf(r) < 0.03125f ? p : (e - 1.0f) * rA;
}

// The same coefficient divided by ln 2, from log2-unit arguments: t = delta A
// / ln 2, dl = delta / ln 2, e = exp2(t) and rAl = 1 / (A ln 2) (0 when A =
// 0); the series is the one above with r = t ln 2 and the same cut.
__device__ __forceinline__ float zoh_coef_l2(float t, float dl, float e, float rAl) {
  constexpr float c1 = 0.5f * kLn2, c2 = kLn2 * kLn2 / 6, c3 = kLn2 * kLn2 * kLn2 / 24;
  const float p = dl * fmaf(t, fmaf(t, fmaf(t, c3, c2), c1), 1.0f);
  return fabsf(t) < 0.03125f * kLog2e ? p : (e - 1.0f) * rAl;
}

// ---------------------------------------------------------------- io

typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 is the upper half of an IEEE binary32.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats to bf16 (round to nearest even), lo in the low half: one
// conversion of the pair.
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){lo, hi}, bf16x2v));
}

template <typename IO>
struct Io;

template <>
struct Io<float> {
  static constexpr int V = 4;  // elements per 16-byte access
  __device__ static float ld1(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
  __device__ static void ldv(const void* p, int64_t i, float* o) {
    const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
  __device__ static void st1(void* p, int64_t i, float v) { static_cast<float*>(p)[i] = v; }
  __device__ static void stv(void* p, int64_t i, const float* v) {
    *reinterpret_cast<float4*>(static_cast<float*>(p) + i) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

template <>
struct Io<uint16_t> {  // bf16 bit patterns
  static constexpr int V = 8;
  __device__ static float ld1(const void* p, int64_t i) {
    return __uint_as_float((uint32_t) static_cast<const uint16_t*>(p)[i] << 16);
  }
  __device__ static void ldv(const void* p, int64_t i, float* o) {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
    o[0] = bf_lo(v.x); o[1] = bf_hi(v.x); o[2] = bf_lo(v.y); o[3] = bf_hi(v.y);
    o[4] = bf_lo(v.z); o[5] = bf_hi(v.z); o[6] = bf_lo(v.w); o[7] = bf_hi(v.w);
  }
  __device__ static void st1(void* p, int64_t i, float v) {
    const __bf16 h = (__bf16)v;
    static_cast<uint16_t*>(p)[i] = __builtin_bit_cast(uint16_t, h);
  }
  __device__ static void stv(void* p, int64_t i, const float* v) {
    uint4 w;
    w.x = pack_bf16x2(v[0], v[1]); w.y = pack_bf16x2(v[2], v[3]);
    w.z = pack_bf16x2(v[4], v[5]); w.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p) + i) = w;
  }
};

// Raw buffer accesses: a 32-bit byte offset from a base whose extent is
// given, and reads past the extent return zero, so addresses need no clamps.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_ld128(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint2 buf_ld64(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t buf_ld16(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ void buf_st64(uint2 v, Rsrc r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, v), r, voff, soff, 0);
}
__device__ __forceinline__ void buf_st16(uint32_t v, Rsrc r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t buf_ld32(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ void buf_st32(uint32_t v, Rsrc r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, soff, 0);
}

// ---------------------------------------------------------------- cross-lane

// DPP move: lanes whose source lies outside the pattern, or whose row is
// masked off, receive `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL,
                                                    ROW_MASK, 0xf, false));
}

// DPP move reading 0 where there is no source lane (bound_ctrl).
template <int CTRL>
__device__ __forceinline__ float dpp0(float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(src), CTRL, 0xf, 0xf, true));
}

constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143, kWaveShr1 = 0x138;

// Inclusive scan of (A, H) pairs within each 16-lane row, where (A_prev,
// H_prev) then (A, H) composes to (A_prev A, A H_prev + H).  Hillis-Steele
// with the neighbour's H read through DPP inside the fma (v_fmac_f32_dpp);
// a lane without a source reads H_prev = 0 and keeps H.  A lane without a
// source also zeroes its A, which no later step of the row reads.  On return
// H is exact on every lane (A is not returned).  Each s_nop 1 covers the
// two wait states a DPP read needs after a VALU write of the same register,
// including for code that follows the block.
__device__ __forceinline__ void row_scan16(float A, float& H) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:1 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shr:1 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:2 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shr:2 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:4 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shr:4 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1"
      : "+v"(H), "+v"(A));
}

// The same scan run towards lower lanes (row_shl): on return H on lane l
// composes the pairs of lanes l..15 of its row, i.e. the suffix scan used by
// the adjoint recurrence, which runs backwards in time.
__device__ __forceinline__ void row_scan16_rev(float A, float& H) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shl:1 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shl:1 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shl:2 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shl:2 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shl:4 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shl:4 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shl:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1"
      : "+v"(H), "+v"(A));
}

constexpr int kRowShl1 = 0x101;

// Step across rows (row broadcast) for groups wider than a row: every lane of
// the receiving rows uses its own A, so A keeps the identity where there is
// no source.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void bcast_step(float& A, float& H) {
  const float As = dpp<CTRL, ROW_MASK>(1.0f, A);
  const float Hs = dpp<CTRL, ROW_MASK>(0.0f, H);
  H = fmaf(A, Hs, H);
  A = A * As;
}

// Inclusive scan of (A, H) pairs over each group of LPC consecutive lanes;
// H is exact on every lane on return.
template <int LPC>
__device__ __forceinline__ void group_scan(float A, float& H) {
  if constexpr (LPC == 16) {
    row_scan16(A, H);
  } else {
    bcast_step<kRowShr1, 0xf>(A, H);
    bcast_step<kRowShr2, 0xf>(A, H);
    bcast_step<kRowShr4, 0xf>(A, H);
    bcast_step<kRowShr8, 0xf>(A, H);
    bcast_step<kRowBcast15, 0xa>(A, H);
    if constexpr (LPC >= 64) bcast_step<kRowBcast31, 0xc>(A, H);
  }
}

// H of the previous lane of the group (0 on the group's first lane).
template <int LPC>
__device__ __forceinline__ float group_prev0(float v, bool first) {
  if constexpr (LPC == 16) {
    return dpp0<kRowShr1>(v);
  } else {
    const float p = dpp<kWaveShr1, 0xf>(0.0f, v);
    return first ? 0.0f : p;
  }
}

// Sum over the four 16-lane rows of a wave of eight values per lane.  permlane32_swap trades the upper half of its first operand for
// the lower half of its second, permlane16_swap the odd rows of the first for
// the even rows of the second; adding each swapped pair halves the rows to sum
// while packing two values into one register.  On return row r of lo holds
// the four-row sum of v[red_step(r)] and row r of hi that of v[4 + red_step(r)].
__device__ __forceinline__ int red_step(int row) { return ((row & 1) << 1) | (row >> 1); }

__device__ __forceinline__ void rows_sum8(const float* v, float& lo, float& hi) {
  float s[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[2 * p]),
                                                    __float_as_uint(v[2 * p + 1]), false, false);
    s[p] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  }
  const auto y0 = __builtin_amdgcn_permlane16_swap(__float_as_uint(s[0]), __float_as_uint(s[1]),
                                                   false, false);
  const auto y1 = __builtin_amdgcn_permlane16_swap(__float_as_uint(s[2]), __float_as_uint(s[3]),
                                                   false, false);
  lo = __uint_as_float(y0[0]) + __uint_as_float(y0[1]);
  hi = __uint_as_float(y1[0]) + __uint_as_float(y1[1]);
}

// ---------------------------------------------------------------- forward scan

// Raw (undecoded) storage of K consecutive elements.
template <typename IO, int K>
struct Run;
template <int K>
struct Run<uint16_t, K> {
  uint4 v[K / 8];
  __device__ void unpack(float* o) const {
#pragma unroll
    for (int i = 0; i < K / 8; ++i) {
      o[8 * i + 0] = bf_lo(v[i].x); o[8 * i + 1] = bf_hi(v[i].x);
      o[8 * i + 2] = bf_lo(v[i].y); o[8 * i + 3] = bf_hi(v[i].y);
      o[8 * i + 4] = bf_lo(v[i].z); o[8 * i + 5] = bf_hi(v[i].z);
      o[8 * i + 6] = bf_lo(v[i].w); o[8 * i + 7] = bf_hi(v[i].w);
    }
  }
};
template <int K>
struct Run<float, K> {
  float4 v[K / 4];
  __device__ void unpack(float* o) const {
#pragma unroll
    for (int i = 0; i < K / 4; ++i) {
      o[4 * i + 0] = v[i].x; o[4 * i + 1] = v[i].y; o[4 * i + 2] = v[i].z; o[4 * i + 3] = v[i].w;
    }
  }
};

// r <- p[base + t .. base + t + K), zero past L or when !valid.  VEC: rows
// are 16-byte aligned, so whole runs load as 16-byte vectors.  INB: the
// caller knows that t + K <= L.
template <typename IO, int K, bool VEC, bool INB = false>
__device__ __forceinline__ void run_load(Run<IO, K>& r, const void* p, int64_t base, int64_t t,
                                         int64_t L, bool valid) {
  using VT = typename std::remove_reference<decltype(r.v[0])>::type;
  constexpr int V = Io<IO>::V;
  if (VEC && valid && (INB || t + K <= L)) {
    const VT* q = reinterpret_cast<const VT*>(static_cast<const IO*>(p) + base + t);
#pragma unroll
    for (int i = 0; i < K / V; ++i) r.v[i] = q[i];
  } else {
    IO e[K];
#pragma unroll
    for (int i = 0; i < K; ++i)
      e[i] = (valid && t + i < L) ? static_cast<const IO*>(p)[base + t + i] : IO(0);
    __builtin_memcpy(&r.v[0], e, sizeof e);
  }
}

template <typename IO, int K, bool VEC, bool INB = false>
__device__ __forceinline__ void run_store(void* p, int64_t base, int64_t t, int64_t L,
                                          bool valid, const float* v) {
  if (!valid) return;
  if (VEC && (INB || t + K <= L)) {
#pragma unroll
    for (int i = 0; i < K; i += Io<IO>::V) Io<IO>::stv(p, base + t + i, v + i);
  } else {
#pragma unroll
    for (int i = 0; i < K; ++i)
      if (t + i < L) Io<IO>::st1(p, base + t + i, v[i]);
  }
}

struct ScanArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  const void* z;
  const float* delta_bias;
  const float* h0;
  void* y;
  float* final_state;
  int64_t dim, dstate, seqlen;
  int softplus;
  float* ckpt;  // or null: state entering every kCkptT-step block, [batch, dim, ceil(L / kCkptT), dstate]
};

// Discretization rules (the bbar_mode of the C ABI): Abar = exp(delta A) with
// Bbar = delta B or the exact ZOH input (A^-1 (exp(delta A) - 1) B); Euler,
// Abar = 1 + delta A, Bbar = delta B; bilinear, Abar = (1 + delta A / 2) /
// (1 - delta A / 2), Bbar = delta B / (1 - delta A / 2) ("State-space
// models", section "Discretization").
constexpr int kRuleDeltaB = 0, kRuleZoh = 1, kRuleEuler = 2, kRuleBilinear = 3;

// LDS of one CU on gfx950 (the most one workgroup can hold).
constexpr size_t kLdsBytes = 160 * 1024;

// Steps between the states that the checkpoint pass keeps for the backward.
constexpr int kCkptT = 128;

// CKPT: the pass that the backward recomputes from: it writes the state
// entering every kCkptT-step block to a.ckpt and computes no output.
template <typename IO, int LPC, int K, int W, int NT, bool VEC, int RULE, bool GATE,
          bool CKPT = false>
__global__ void __launch_bounds__(64 * W)
    __attribute__((amdgpu_waves_per_eu(LPC == 16 && SELSCAN_WAVES_PER_EU ? SELSCAN_WAVES_PER_EU : 1)))
    scan_fwd_kernel(const ScanArgs a) {
  constexpr int CPW = 64 / LPC;  // channels per wave
  constexpr int CPB = CPW * W;   // channels per workgroup
  constexpr int T = LPC * K;     // timesteps per chunk
  constexpr int KP = K + 4;      // padded per-lane run in LDS (spreads banks)
  constexpr int V = Io<IO>::V;
  constexpr int TV = T / V;      // staged vectors per B/C row
  constexpr int NTH = 64 * W;
  constexpr int ITEMS = (2 * NT * TV + NTH - 1) / NTH;  // staged vectors per thread
  static_assert(K % V == 0 && K % 4 == 0, "K must be a multiple of the vector width");
  __shared__ float4 sB4[NT * LPC * KP / 4];
  __shared__ float4 sC4[NT * LPC * KP / 4];
  extern __shared__ float sDyn[];  // [CPB][dstate] carry, then [CPB][dstate] A
  float* sB = reinterpret_cast<float*>(sB4);
  float* sC = reinterpret_cast<float*>(sC4);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int seg = lane % LPC;
  const bool first = seg == 0;
  const int chb = wave * CPW + lane / LPC;
  const int64_t b = blockIdx.y;
  const int64_t d0 = (int64_t)blockIdx.x * CPB;
  const int64_t d = d0 + chb;
  // Lanes of a channel past `dim` compute on channel 0's data in their own
  // lane group and store nothing.
  const bool dvalid = d < a.dim;
  const int64_t N = a.dstate, L = a.seqlen;
  const int64_t row = (b * a.dim + (dvalid ? d : 0)) * L;
  const int64_t bcrow = b * N * L;

  float* sCarry = sDyn;
  float* sA = sDyn + CPB * N;
  for (int64_t i = threadIdx.x; i < CPB * N; i += NTH) {
    const int64_t c = i / N, n = i % N;
    const bool ok = d0 + c < a.dim;
    const float h0v = (a.h0 && ok) ? a.h0[(b * a.dim + d0 + c) * N + n] : 0.0f;
    sCarry[i] = h0v * kLog2e;  // h / ln 2 (below)
    sA[i] = ok ? a.A[(d0 + c) * N + n] : 0.0f;
    // the checkpoint of block 0 is h0 itself
    if (a.ckpt && ok) a.ckpt[(b * a.dim + d0 + c) * ((L + kCkptT - 1) / kCkptT) * N + n] = h0v;
  }
  // y accumulates (D u + C h) / ln 2 (see below)
  const float Dl = ((a.Dskip && dvalid) ? a.Dskip[d] : 0.0f) * kLog2e;
  const float bias = ((a.delta_bias && dvalid) ? a.delta_bias[d] : 0.0f) * kLog2e;  // bias / ln 2
  float* carry_row = sCarry + chb * N;
  const float* a_row = sA + chb * N;

  // B, C rows [n0, n0 + nt) x [t0, t0 + T) -> LDS as float32, laid out so
  // that each lane reads its K steps as contiguous float4s.  FULL: nt = NT
  // and the chunk lies inside [0, L) (the index arithmetic is then by
  // constants).
  auto stage_bc = [&](int64_t t0, int64_t n0, int nt_arg, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int nt = FULL ? NT : nt_arg;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int item = threadIdx.x + k * NTH;
      if (item < 2 * nt * TV) {
        const int tensor = item / (nt * TV);
        const int r = item % (nt * TV);
        const int nl = r / TV, tloc = (r % TV) * V;
        Run<IO, V> rv;
        run_load<IO, V, VEC, FULL>(rv, tensor ? a.Cm : a.Bm, bcrow + (n0 + nl) * L, t0 + tloc, L, true);
        float v[V];
        rv.unpack(v);
        float* dst = (tensor ? sC : sB) + (nl * LPC + tloc / K) * KP + tloc % K;
#pragma unroll
        for (int q = 0; q < V; q += 4)
          *reinterpret_cast<float4*>(dst + q) = make_float4(v[q], v[q + 1], v[q + 2], v[q + 3]);
      }
    }
  };

  // PREF (the layouts with 32 and 64 lanes per channel, whose occupancy the
  // grid limits to one or two workgroups per CU; vectorised bf16 rows: a
  // float32 tile is twice the registers, which spill there): the next
  // B/C tile is loaded into registers while the current one is computed,
  // instead of between two barriers where every wave of the workgroup waits
  // for it.  The loads are unconditional (a vector past L reads its row's
  // start instead; rows are whole vectors long) and the vectors past L are
  // zeroed when the tile is written to LDS, so the number of memory
  // operations is the same on every path and the compiler's wait for the
  // tile covers only older ones.
  constexpr bool PREF = LPC >= 32 && VEC && !CKPT && sizeof(IO) == 2;
  uint4 pre[PREF ? ITEMS : 1];
  int64_t pre_t0 = 0;  // first step of the prefetched tile's chunk
  auto tile_nt = [&](int64_t n0) { return (int)((N - n0) < NT ? (N - n0) : NT); };
  auto fetch_bc = [&](int64_t t0, int64_t n0) __attribute__((always_inline)) {
    const int nt = tile_nt(n0);
    pre_t0 = t0;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      // items past the tile (a last tile of fewer states) load item 0's vector
      const int item0 = threadIdx.x + k * NTH;
      const int item = item0 < 2 * nt * TV ? item0 : 0;
      const int tensor = item / (nt * TV);
      const int r = item % (nt * TV);
      const int nl = r / TV, tloc = (r % TV) * V;
      const int64_t rowp = bcrow + (n0 + nl) * L;
      const int64_t t = t0 + tloc < L ? t0 + tloc : 0;
      pre[k] = *reinterpret_cast<const uint4*>(static_cast<const IO*>(tensor ? a.Cm : a.Bm) + rowp + t);
    }
  };
  auto put_bc = [&](int64_t n0) __attribute__((always_inline)) {
    const int nt = tile_nt(n0);
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int item = threadIdx.x + k * NTH;
      if (item < 2 * nt * TV) {
        const int tensor = item / (nt * TV);
        const int r = item % (nt * TV);
        const int nl = r / TV, tloc = (r % TV) * V;
        Run<IO, V> rv;
        const bool in = pre_t0 + tloc < L;
        const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
        __builtin_memcpy(&rv.v[0], in ? &pre[k] : &z4, sizeof(uint4));
        float v[V];
        rv.unpack(v);
        float* dst = (tensor ? sC : sB) + (nl * LPC + tloc / K) * KP + tloc % K;
#pragma unroll
        for (int q = 0; q < V; q += 4)
          *reinterpret_cast<float4*>(dst + q) = make_float4(v[q], v[q + 1], v[q + 2], v[q + 3]);
      }
    }
  };
  // write the prefetched tile (t0, n0) and fetch the one after it: the next
  // states of the chunk, else the next chunk's first (past L: not read)
  auto put_and_fetch = [&](int64_t t0, int64_t n0) __attribute__((always_inline)) {
    put_bc(n0);
    asm volatile("" ::: "memory");  // the new loads stay after the old tile is consumed
    if (n0 + NT < N) fetch_bc(t0, n0 + NT);
    else fetch_bc(t0 + T < L ? t0 + T : t0, 0);
  };

  // One chunk of T timesteps.  FULL: the chunk lies inside [0, L) and N is a
  // multiple of NT, so no step or state needs masking.
  auto chunk = [&](int64_t t0, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int64_t tl = t0 + seg * K;
    // Step sizes are kept in log2 units, dl = delta / ln 2 (from the raw
    // step by one fma), so that Abar = exp(delta A) = exp2(dl A) with A in
    // natural units.  The u weight dl u = delta u / ln 2 scales the whole
    // recurrence: lanes, carries and the readout hold h / ln 2 and y / ln 2,
    // converted where a state enters (h0) or leaves (final state,
    // checkpoints) and once per output step (for free inside the gate).
    float dl[K], w[K], y[K], ul[K];
    float S = 0.0f;
    // issue this chunk's sequence loads first: they complete while the first
    // B/C tile is staged.  With PREF every lane loads (lanes of channels past
    // `dim` read channel 0's row and store nothing), so that the number of
    // loads is fixed and the wait for the prefetched tile need not cover them.
    const bool lv = PREF ? true : dvalid;
    Run<IO, K> ru, rd, rz;
    run_load<IO, K, VEC, FULL>(ru, a.u, row, tl, L, lv);
    run_load<IO, K, VEC, FULL>(rd, a.delta, row, tl, L, lv);
    if constexpr (GATE) run_load<IO, K, VEC, FULL>(rz, a.z, row, tl, L, lv);
    __syncthreads();  // every wave is done with the previous chunk's last tile
    if constexpr (PREF) put_and_fetch(t0, 0);
    else stage_bc(t0, 0, (int)(N < NT ? N : NT), full_tag);
    __syncthreads();
    {
      float raw[K];
      ru.unpack(ul);
      rd.unpack(raw);
#pragma unroll
      for (int i = 0; i < K; ++i) {
        const float xl = fmaf(raw[i], kLog2e, bias);  // (raw + bias) / ln 2
        float v = a.softplus ? softplus_xl(xl) : xl;
        if constexpr (!FULL) v = (tl + i < L) ? v : 0.0f;  // identity step past the end
        dl[i] = v;
        w[i] = v * ul[i];
        y[i] = Dl * ul[i];
        S += v;
      }
    }

    // one state n: discretize, fold, scan, apply, read out
    auto state = [&](int j, int64_t n) {
      const float An = a_row[n];
      const float c = carry_row[n];  // state at the chunk start
      const float* pb = sB + (j * LPC + seg) * KP;
      const float* pc = sC + (j * LPC + seg) * KP;
      float av[K], xv[K];
      const float rA = (RULE == kRuleZoh && An != 0.0f) ? rcp(An * kLn2) : 0.0f;  // 1 / (A ln 2)
#pragma unroll
      for (int i = 0; i < K; i += 4) {
        const float4 bb = *reinterpret_cast<const float4*>(pb + i);
        const float bq[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (RULE == kRuleDeltaB) {
            av[i + q] = ex2(dl[i + q] * An);
            xv[i + q] = w[i + q] * bq[q];
          } else if constexpr (RULE == kRuleZoh) {
            const float t = dl[i + q] * An;  // delta A / ln 2
            av[i + q] = ex2(t);
            xv[i + q] = zoh_coef_l2(t, dl[i + q], av[i + q], rA) * bq[q] * ul[i + q];  // / ln 2, as h
          } else if constexpr (RULE == kRuleEuler) {
            av[i + q] = fmaf(dl[i + q] * kLn2, An, 1.0f);
            xv[i + q] = w[i + q] * bq[q];
          } else {  // bilinear
            const float x = 0.5f * kLn2 * dl[i + q] * An;  // delta A / 2
            const float r = rcp(1.0f - x);
            av[i + q] = (1.0f + x) * r;
            xv[i + q] = w[i + q] * r * bq[q];
          }
        }
      }
      // fold the lane's K steps into one pair; the channel's first lane starts
      // from the carried state, the others from zero, so the scan below hands
      // every lane its exact incoming state
      float H = fmaf(av[0], first ? c : 0.0f, xv[0]);
#pragma unroll
      for (int i = 1; i < K; ++i) H = fmaf(av[i], H, xv[i]);
      // product of the lane's K decays
      float Al;
      if constexpr (RULE <= kRuleZoh) {
        Al = ex2(An * S);
      } else {
        Al = av[0];
#pragma unroll
        for (int i = 1; i < K; ++i) Al *= av[i];
      }
      group_scan<LPC>(Al, H);
      const float He = group_prev0<LPC>(H, first);
      float h = first ? c : He;
      if (seg == LPC - 1) carry_row[n] = H;
      static_assert(!CKPT || (kCkptT % K == 0 && T % kCkptT == 0), "checkpoints fall on lane starts");
      if constexpr (kCkptT % K == 0 && T % kCkptT == 0) {
        if (a.ckpt && dvalid && (seg * K) % kCkptT == 0 && tl < L && tl > 0)  // block 0's: above
          a.ckpt[((b * a.dim + d) * ((L + kCkptT - 1) / kCkptT) + tl / kCkptT) * N + n] = h * kLn2;
      }
#pragma unroll
      for (int i = 0; i < K; i += 4) {
        const float4 cc = *reinterpret_cast<const float4*>(pc + i);
        const float cq[4] = {cc.x, cc.y, cc.z, cc.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          h = fmaf(av[i + q], h, xv[i + q]);
          if constexpr (!CKPT) y[i + q] = fmaf(cq[q], h, y[i + q]);
        }
      }
    };

    for (int64_t n0 = 0; n0 < N; n0 += NT) {
      if (n0 > 0) {
        __syncthreads();  // every wave is done with the previous tile
        if constexpr (PREF) put_and_fetch(t0, n0);
        else stage_bc(t0, n0, (int)((N - n0) < NT ? (N - n0) : NT), full_tag);
        __syncthreads();
      }
      const int nt = FULL ? NT : (int)((N - n0) < NT ? (N - n0) : NT);
#pragma unroll 1
      for (int j = 0; j < nt; ++j) state(j, n0 + j);
    }
    if constexpr (CKPT) return;
    if constexpr (GATE) {
      float zz[K];
      rz.unpack(zz);
#pragma unroll
      for (int i = 0; i < K; ++i) y[i] *= silu_ln2(zz[i]);
    } else {
#pragma unroll
      for (int i = 0; i < K; ++i) y[i] *= kLn2;
    }
    run_store<IO, K, VEC, FULL>(a.y, row, tl, L, dvalid, y);
  };

  if constexpr (PREF) fetch_bc(0, 0);
  int64_t t0 = 0;
  if (N % NT == 0) {
    for (; t0 + T <= L; t0 += T) chunk(t0, std::true_type{});
  }
  for (; t0 < L; t0 += T) chunk(t0, std::false_type{});

  if (a.final_state && dvalid) {
    // each channel's carry was written by its own wave; LDS is in order per wave
    for (int64_t n = seg; n < N; n += LPC)
      a.final_state[(b * a.dim + d) * N + n] = carry_row[n] * kLn2;
  }
}

// ---------------------------------------------------------------- forward scan, time-pipelined (16 states)

// Four consecutive bf16 elements of a row (one lane's steps), packed.
struct Quad {
  uint2 v;
  __device__ float at(int i) const {
    const uint32_t w = i < 2 ? v.x : v.y;
    return (i & 1) ? bf_hi(w) : bf_lo(w);
  }
};

// A quad of a row read through a buffer resource at byte offset voff + soff;
// only its first n elements are read (n <= 0: none), the rest are zero.  VEC:
// one aligned 8-byte load (L is a multiple of 8 and a quad starts at a
// multiple of 4, so it lies wholly before the row's end or wholly past it).
template <bool VEC>
__device__ __forceinline__ void quad_load(Quad& q, Rsrc rs, uint32_t voff, uint32_t soff, int n) {
  if (VEC) {
    q.v = n >= 4 ? buf_ld64(rs, voff, soff) : make_uint2(0u, 0u);
  } else {
    uint32_t e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = i < n ? buf_ld16(rs, voff + 2 * i, soff) : 0u;
    q.v = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
  }
}

// Makes the compiler treat a loaded quad as unknown until this point, so the
// wait for its load stays here instead of moving up to the load.
__device__ __forceinline__ void opaque(Quad& q) { asm volatile("" : "+v"(q.v.x), "+v"(q.v.y)); }

// Orders this lane's LDS accesses before and after it for the compiler; the
// hardware already runs one wave's LDS instructions in order, so this is what
// lanes of one wave need to exchange data through LDS.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Forward scan for 16 states and bf16 rows in which every lane runs the
// recurrence in time order over its own steps, with no fold, scan or replay:
// each element costs its discretization, one state fma and one readout fma
// (the recurrent form, "State-space models", section "Recurrence and
// convolution"), against one more fma plus the scan for the kernel above.
//
// A workgroup holds 16 channels of one sequence and four waves; wave s owns
// time segment s (16 steps) of every 64-step chunk.  In a wave, lane 16 r + c
// holds channel c and the states n = 4 j + r, one after another (j = 0..3:
// four "items" per chunk).  The waves form a ring over time: wave s runs item
// (chunk t, j) from the state that wave s - 1 handed over for the same item
// (for s = 0: wave 3, chunk t - 1) through an LDS slot, and counts its handed
// items in LDS; a wave waits only for its predecessor's count (a bounded
// spin), so the four segments of a chunk run concurrently, each one item
// behind the other.  Each chunk's B and C rows of a segment are staged by the
// wave that uses them.
//
// Per-step work (softplus step size, u weight, D u, gate) is done once per
// (channel, step): lane (r, c) prepares steps 4 r .. 4 r + 3 of its channel's
// segment of the next chunk during the items of this one, and the wave shares
// them through LDS.  Each lane's readout sums over its own 4 states; after
// the last item of a chunk the 4 rows are added with lane swaps, lane (r, c)
// finishes steps 4 r .. 4 r + 3 into an LDS copy of the chunk's y, and the
// last wave stores the chunk's y rows whole (128 bytes each) once every wave
// has written its segment, so no line of y is written in pieces.
//
// Registers are held to 96 (five waves per SIMD: 20480 channels give exactly
// five workgroups per CU) and LDS to 30 KiB per workgroup.


// CKPT: the checkpoint pass of the backward (states at every kCkptT-step
// block start to a.ckpt, no output).
template <bool VEC, int RULE, bool GATE, bool CKPT = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5)))
    scan_fwd_pipe_kernel(const ScanArgs a) {
  using IO = uint16_t;
  static_assert(RULE != kRuleZoh, "exact ZOH needs more registers than five waves per SIMD leave");
  constexpr int W = 4;      // waves = time segments of a chunk
  constexpr int K = 16;     // steps per segment
  constexpr int T = W * K;  // steps per chunk
  constexpr int NS = 16;    // states
  constexpr int KP = K + 4; // padded LDS rows (spreads banks)
  static_assert(kCkptT % T == 0, "checkpoint blocks are whole chunks");
  // per wave: the B and C rows of its segment, [2][NS][KP]
  __shared__ float4 sWave[W][2 * NS * KP / 4];
  // the chunk's y as bf16, [chunk parity][16 channels][64 steps + 8 pad],
  // stored to HBM as whole 128-byte rows by the last wave
  __shared__ __align__(16) uint16_t sY[2][16][T + 8];
  // per wave: step sizes and u weights of its segment, [2][16 channels][KP]
  __shared__ float4 sPrep[W][2 * 16 * KP / 4];
  // state handed from wave s to wave s + 1, [s][j][lane] for the states
  // n = 4 j + r of lane 16 r + c (the ring's dependences keep a slot from
  // being rewritten before it is read; wave 3's slots start with the initial
  // state), and the number of items each wave has handed over
  __shared__ float sCarry[W][4][64];
  __shared__ int sDone[W];
  // A as [j][lane]
  __shared__ float sA[4][64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane >> 4, cl = lane & 15;
  const int64_t b = blockIdx.y;
  const int64_t d0 = (int64_t)blockIdx.x * 16;
  const int64_t d = d0 + cl;
  // lanes of a channel past `dim` compute on channel d0 and store nothing
  const bool dvalid = d < a.dim;
  const int64_t dc = dvalid ? d : d0;
  const int64_t L = a.seqlen;
  const int nchunks = (int)((L + T - 1) / T);  // L < 2^26 (launcher)
  float* tile = reinterpret_cast<float*>(sWave[wave]);
  float* prep = reinterpret_cast<float*>(sPrep[wave]);
  const int seg0 = K * wave;  // first step of this wave's segment in a chunk
  // Buffer resources over the rows of the workgroup's channels and of the
  // sequence's B and C (the launcher checks that 16 L elements span less
  // than 2^31 bytes): a lane adds its own byte offset, the chunk a uniform
  // one.  Reads past a row's end within the last chunk are masked per lane.
  constexpr int ES = sizeof(IO);
  const int64_t seq_base = (b * a.dim + d0) * L;
  const int64_t nrows = a.dim - d0 < 16 ? a.dim - d0 : 16;
  const int seq_bytes = (int)(nrows * L * ES);
  const Rsrc u_r = make_rsrc(static_cast<const IO*>(a.u) + seq_base, seq_bytes);
  const Rsrc dl_r = make_rsrc(static_cast<const IO*>(a.delta) + seq_base, seq_bytes);
  const Rsrc z_r = make_rsrc(GATE ? static_cast<const IO*>(a.z) + seq_base : nullptr, GATE ? seq_bytes : 0);
  const Rsrc y_r = make_rsrc(static_cast<IO*>(a.y) + seq_base, seq_bytes);
  const int bc_bytes = (int)(NS * L * ES);
  const Rsrc B_r = make_rsrc(static_cast<const IO*>(a.Bm) + b * NS * L, bc_bytes);
  const Rsrc C_r = make_rsrc(static_cast<const IO*>(a.Cm) + b * NS * L, bc_bytes);
  const int qstep = seg0 + 4 * r;  // first step of this lane's quad in a chunk
  // Lane (r, c) reads its quad of channel c's rows and, for the staging of
  // the B and C tile, the same quad of state c's rows: one offset.  Rows of
  // channels past `dim` lie past the resource's extent and read as zero.
  const uint32_t seq_off = (uint32_t)((cl * L + qstep) * ES);

  // Step sizes are kept in log2 units (dl = delta / ln 2, from the raw step
  // by one fma), so that Abar = exp2(dl A) for the delta*B rule; A is held
  // as A ln 2 for the other rules, whose formulas take delta A.  The u weight
  // dl u = delta u / ln 2 then scales the whole recurrence: the lanes carry
  // h / ln 2, which is converted where a state enters (h0) or leaves (final
  // state, checkpoints), and the readout sum is multiplied by ln 2 once per
  // step, for free inside the gate's reciprocal.
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float Av = a.A[dc * NS + 4 * j + r];
      sA[j][lane] = RULE == kRuleDeltaB ? Av : Av * kLn2;
    }
  }
  const float Dv = (a.Dskip && dvalid) ? a.Dskip[d] * kLog2e : 0.0f;  // D / ln 2
  const float bias = (a.delta_bias && dvalid) ? a.delta_bias[d] * kLog2e : 0.0f;  // bias / ln 2

  // steps of chunk c before L (uniform, at most T), and the byte offset of
  // the chunk.  The chunk body below comes in two forms: FULL for chunks c
  // with c + 2 < L / T (this chunk and the two it loads ahead hold T steps,
  // so no lane masks its loads or steps), and the general one for the rest.
  auto left = [&](int c) { return (int)(L - (int64_t)c * T < T ? L - (int64_t)c * T : T); };
  auto coff = [&](int c) { return (uint32_t)c * (uint32_t)(T * ES); };
  // elements of the lane's quad before L in chunk c
  auto quad_n = [&](int c, auto full) { return decltype(full)::value ? 4 : left(c) - qstep; };
  // u and delta of the lane's quad of a chunk
  struct Ud {
    Quad u, dl;
  };
  auto load_ud = [&](Ud& q, int c, auto full) {
    const int n = quad_n(c, full);
    quad_load<VEC>(q.u, u_r, seq_off, coff(c), n);
    quad_load<VEC>(q.dl, dl_r, seq_off, coff(c), n);
  };
  Quad bq_raw, cq_raw;
  auto load_bc = [&](int c, auto full) {
    const int n = quad_n(c, full);
    quad_load<VEC>(bq_raw, B_r, seq_off, coff(c), n);
    if constexpr (!CKPT) quad_load<VEC>(cq_raw, C_r, seq_off, coff(c), n);
  };
  // step size (log2 units) and u weight of step i of this lane's quad
  auto prep_step = [&](const Ud& q, int i, int c, auto full, float& dlo, float& wo) {
    const float xl = fmaf(q.dl.at(i), kLog2e, bias);  // (raw + bias) / ln 2
    float v = a.softplus ? softplus_xl(xl) : xl;
    if constexpr (!decltype(full)::value) v = qstep + i < left(c) ? v : 0.0f;  // identity step past the end
    dlo = v;
    wo = v * q.u.at(i);  // delta u
  };
  // chunk cc's y rows from sY to HBM: lane 4 k + q writes steps 16 q .. 16 q
  // + 15 of channel k, so four lanes cover one 128-byte row
  auto store_y = [&](int cc, auto full) {
    cc = __builtin_amdgcn_readfirstlane(cc);  // uniform: keeps the offset scalar
    const int sch = lane >> 2, sq = lane & 3;
    if (d0 + sch >= a.dim) return;
    const uint16_t* src = &sY[cc & 1][sch][16 * sq];
    const int n = decltype(full)::value ? 16 : left(cc) - 16 * sq;  // steps of this piece before L
    const uint32_t off = (uint32_t)((sch * L + 16 * sq) * ES);
    if (VEC) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        if (n >= 8 * (h2 + 1))
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int,
                                 *reinterpret_cast<const uint4*>(src + 8 * h2)),
              y_r, off + 16 * h2, coff(cc), 0);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i < n) buf_st16(src[i], y_r, off + 2 * i, coff(cc));
    }
  };
  // steps i, i + 1 of the lane's quad, for the next chunk -> LDS (the wave
  // has read this chunk's values into registers by then)
  auto prep_pair = [&](const Ud& q, int i, int c, auto full) {
    float d0v, w0v, d1v, w1v;
    prep_step(q, i, c, full, d0v, w0v);
    prep_step(q, i + 1, c, full, d1v, w1v);
    *reinterpret_cast<float2*>(prep + cl * KP + 4 * r + i) = make_float2(d0v, d1v);
    *reinterpret_cast<float2*>(prep + 16 * KP + cl * KP + 4 * r + i) = make_float2(w0v, w1v);
  };

  // u of the chunk being finished (for D u), z of it, and u and delta of
  // the next chunk (loaded during the last item of the chunk before)
  const std::false_type general{};
  Ud nxt{};
  Quad cur_u{}, zq{};
  {
    Ud first;
    load_ud(first, 0, general);
    load_bc(0, general);
    if (nchunks > 1) load_ud(nxt, 1, general);
    cur_u = first.u;
    prep_pair(first, 0, 0, general);
    prep_pair(first, 2, 0, general);
  }
  // states: [channel][NS] rows from (b, d0) on; checkpoints: [channel][nblk][NS]
  const int64_t nblk = (L + kCkptT - 1) / kCkptT;
  const int64_t st_base = (b * a.dim + d0) * NS;
  const Rsrc fs_r = make_rsrc(a.final_state ? a.final_state + st_base : nullptr,
                              a.final_state ? (int)(nrows * NS * 4) : 0);
  const Rsrc ck_r = make_rsrc(a.ckpt ? a.ckpt + st_base * nblk : nullptr, a.ckpt ? (int)(nrows * nblk * NS * 4) : 0);
  const uint32_t fs_off = (uint32_t)(((dc - d0) * NS + r) * 4);
  const uint32_t ck_off = (uint32_t)(((dc - d0) * nblk * NS + r) * 4);
  if (wave == W - 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float h0v = (a.h0 && dvalid) ? a.h0[(b * a.dim + d) * NS + 4 * j + r] : 0.0f;
      sCarry[W - 1][j][lane] = h0v * kLog2e;  // h0 / ln 2
    }
  }
  if (a.ckpt && wave == 0 && dvalid) {  // the state entering block 0, exactly h0
#pragma unroll
    for (int j = 0; j < 4; ++j)
      buf_st32(__float_as_uint(a.h0 ? a.h0[(b * a.dim + d) * NS + 4 * j + r] : 0.0f), ck_r, ck_off, 16 * j);
  }
  if (threadIdx.x < W) sDone[threadIdx.x] = 0;
  __syncthreads();
  const int pred = (wave + W - 1) & (W - 1);  // the wave whose states this one continues

  auto chunk = [&](const int c, auto full) {
    constexpr bool FULL = decltype(full)::value;
    const bool more = FULL || c + 1 < nchunks;
    const bool more2 = FULL || c + 2 < nchunks;
    // this chunk's B, C rows of the segment -> LDS; prefetch the next ones.
    // The raw quads stay packed until here, so that the wait for their load
    // (issued a chunk earlier) falls here.
    {
      opaque(bq_raw);
      opaque(cq_raw);
      float* dst = tile + cl * KP + 4 * r;
      *reinterpret_cast<float4*>(dst) = make_float4(bq_raw.at(0), bq_raw.at(1), bq_raw.at(2), bq_raw.at(3));
      if constexpr (!CKPT)
        *reinterpret_cast<float4*>(dst + NS * KP) =
            make_float4(cq_raw.at(0), cq_raw.at(1), cq_raw.at(2), cq_raw.at(3));
    }
    if (more) load_bc(c + 1, full);
    if constexpr (GATE && !CKPT) quad_load<VEC>(zq, z_r, seq_off, coff(c), quad_n(c, full));
    wave_lds_sync();
    float dl[K], w[K], y[K];
#pragma unroll
    for (int i = 0; i < K; i += 4) {
      const float4 p = *reinterpret_cast<const float4*>(prep + cl * KP + i);
      const float4 q = *reinterpret_cast<const float4*>(prep + 16 * KP + cl * KP + i);
      dl[i] = p.x; dl[i + 1] = p.y; dl[i + 2] = p.z; dl[i + 3] = p.w;
      w[i] = q.x; w[i + 1] = q.y; w[i + 2] = q.z; w[i + 3] = q.w;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = 4 * j + r;
      const int item = 4 * c + j;
      // wait until the predecessor has handed over this item's states: wave
      // s - 1 the same item, wave 3 (for wave 0) the item one chunk back
      // (in chunk 0 wave 0 needs at most 0 items: its slots hold h0).
      // The wait polls the count without sleeping (a sleep between polls
      // measured 0.5 % slower) and is bounded (2^23 polls, a fraction of a
      // second); the waves of a workgroup are resident together, so it never
      // runs out in a correct launch, and if it did the kernel would still end.
      {
        const int need = wave == 0 ? item - 3 : item + 1;
#pragma unroll 1
        for (int spin = 0; spin < (1 << 23); ++spin) {
          if (__builtin_amdgcn_readfirstlane(__hip_atomic_load(&sDone[pred], __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_WORKGROUP)) >= need)
            break;
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      }
      float h = sCarry[pred][j][lane];
      if constexpr (!CKPT) {
        // the last wave stores the previous chunk's y: every wave finished it
        // before handing over this chunk's first item
        if (j == 0 && wave == W - 1 && c > 0) store_y(c - 1, full);
      }
      if (a.ckpt && wave == 0 && (c & 1) == 0 && c > 0 && dvalid)  // block 0's is h0 (below)
        buf_st32(__float_as_uint(h * kLn2), ck_r, ck_off, (uint32_t)(((c >> 1) * NS + 4 * j) * 4));
      const float A = sA[j][lane];
      const float* pb = tile + n * KP;
      const float* pc = tile + NS * KP + n * KP;
#pragma unroll
      for (int i = 0; i < K; i += 4) {
        // read B and C four steps at a time (not all up front: registers)
        if (i > 0) asm volatile("" ::: "memory");
        const float4 bb = *reinterpret_cast<const float4*>(pb + i);
        const float4 cc = *reinterpret_cast<const float4*>(pc + i);
        const float bq[4] = {bb.x, bb.y, bb.z, bb.w};
        const float cq[4] = {cc.x, cc.y, cc.z, cc.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float dli = dl[i + q], wi = w[i + q];
          float av, xv;
          if constexpr (RULE == kRuleDeltaB) {
            av = ex2(dli * A);
            xv = wi * bq[q];
          } else if constexpr (RULE == kRuleEuler) {
            av = fmaf(dli, A, 1.0f);
            xv = wi * bq[q];
          } else {  // bilinear
            const float x = 0.5f * dli * A;  // delta A / 2
            const float rr = rcp(1.0f - x);
            av = (1.0f + x) * rr;
            xv = wi * rr * bq[q];
          }
          h = fmaf(av, h, xv);
          if constexpr (!CKPT) y[i + q] = j == 0 ? cq[q] * h : fmaf(cq[q], h, y[i + q]);
        }
      }
      // keep the readout sums current item by item (the compiler would
      // otherwise hold every state of the chunk until the last item)
      if constexpr (!CKPT) {
#pragma unroll
        for (int i = 0; i < K; ++i) asm volatile("" : "+v"(y[i]));
      }
      sCarry[wave][j][lane] = h;
      // one wave's LDS accesses complete in order, so the count lands after
      // the state (a compiler fence keeps that order in the code; no wait)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      if (lane == 0) __hip_atomic_store(&sDone[wave], item + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (wave == W - 1 && !more && a.final_state && dvalid) buf_st32(__float_as_uint(h * kLn2), fs_r, fs_off, 16 * j);
      // the next chunk's step sizes and u weights: two steps after each of
      // the middle items (the first item stages B and C, the last finishes
      // the chunk; this balances the items)
      if (more && (j == 1 || j == 2)) {
        if (j == 1) {
          opaque(nxt.u);
          opaque(nxt.dl);
        }
        prep_pair(nxt, 2 * (j - 1), c + 1, full);
      }
      if (j == 3 && CKPT) {
        if (more2) load_ud(nxt, c + 2, full);
      } else if (j == 3) {
        // readout: add the 4 rows' partial sums, finish and store
        float o[4];
        // across the rows with lane swaps: rows_sum8 leaves in row r the sums
        // of v[red_step(r)] and v[4 + red_step(r)]; red_step is its own
        // inverse, so feeding v[red_step(k)] = y[4 k + i] puts step 4 r + i
        // of the sum in row r
        {
          float va[8], vb[8];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            va[red_step(k)] = y[4 * k];
            va[4 + red_step(k)] = y[4 * k + 1];
            vb[red_step(k)] = y[4 * k + 2];
            vb[4 + red_step(k)] = y[4 * k + 3];
          }
          rows_sum8(va, o[0], o[1]);
          rows_sum8(vb, o[2], o[3]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // (sum + D u / ln 2) ln 2, gated
          o[i] = fmaf(Dv, cur_u.at(i), o[i]);
          o[i] *= GATE ? silu_ln2(zq.at(i)) : kLn2;
        }
        *reinterpret_cast<uint2*>(&sY[c & 1][cl][qstep]) =
            make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        cur_u = nxt.u;
        if (more2) load_ud(nxt, c + 2, full);
      }
    }
  };
  // chunks whose loads ahead are all whole, then the rest
  const int nmain = (int)(L / T) - 2;
  int c = 0;
  for (; c < nmain; ++c) chunk(c, std::true_type{});
  for (; c < nchunks; ++c) chunk(c, general);
  if constexpr (!CKPT) {
    __syncthreads();  // every wave has finished the last chunk
    if (wave == W - 1) store_y(nchunks - 1, general);
  }
}

// ---------------------------------------------------------------- backward
//
// Gradients of the forward scan for the loss sum(dy * y) + sum(dfinal * h_L)
// by reverse-mode differentiation of the recurrence, with the states
// recomputed instead of stored ("State-space models", section "The parallel
// scan": the fused kernel recomputes the expanded state in the backward
// pass).  With s = silu(z), dyc = dy s and lambda_t = dL/dh_t:
//
//   lambda_t = dyc_t C_t + Abar_{t+1} lambda_{t+1}        (adjoint, backwards in t)
//   dC_t += dyc_t h_t,  dB_t += lambda_t bbar_t u_t,  du_t = dyc_t D + sum_n lambda_t bbar_t B_t
//   ddelta_t = sum_n [lambda_t h_{t-1} Abar_t A + lambda_t B_t u_t dbbar/ddelta]
//   dA += lambda_t h_{t-1} Abar_t delta_t + lambda_t B_t u_t dbbar/dA
//   draw_t = ddelta_t sigmoid(raw_t + bias),  dz_t = dy_t yc_t silu'(z_t),  dh0 = Abar_0 lambda_0
//
// The adjoint is the same linear recurrence run backwards, so it scans with
// the same pair composition.  Three passes over chunks of T = 16 K steps:
//  1. the forward kernel in checkpoint mode stores the state at every chunk
//     start;
//  2. scan_bwd_carry_kernel runs the adjoint backwards over the chunks of
//     each channel, keeping only mu = Abar lambda at every chunk end (the
//     adjoint that enters the chunk from its future);
//  3. scan_bwd_main_kernel treats every (sequence, chunk) independently,
//     for a run of channel groups: it recomputes the chunk's states from the
//     checkpoint, runs the adjoint from the stored carry and accumulates the
//     gradients; dB and dC, which sum over the channels of a sequence, are
//     summed in registers over the channels a workgroup visits before one
//     global atomic add per value.

// K step sizes in log2 units, in place: softplus(raw + bias) / ln 2, or
// (raw + bias) / ln 2.  One branch around the whole run, so that the K
// softplus chains (two transcendentals each) interleave.
template <int K>
__device__ __forceinline__ void step_log2(float (&v)[K], float bias, int softplus) {
  if (softplus) {
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] = softplus_log2(v[i] + bias);
  } else {
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] = (v[i] + bias) * kLog2e;
  }
}

// exp(r) - 1 for the exact zero-order-hold rule in the gradient kernel, `e`
// being exp(r): a Taylor polynomial where e - 1 would cancel.  The gradient
// kernel keeps this form rather than zoh_coef: at its two-waves-per-SIMD
// register limit that one measured 4 % slower there.
__device__ __forceinline__ float expm1_f(float r, float e) {
  const float p = r * (1.0f + r * (0.5f + r * (1.0f / 6 + r * (1.0f / 24 + r * (1.0f / 120)))));
  return fabsf(r) < 0.03125f ? p : e - 1.0f;
}

// largest state size the backward takes: states are processed in tiles of 16
constexpr int kBwdMaxN = 64;

struct BwdArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  const void* z;
  const float* delta_bias;
  const void* dy;
  const float* dfinal;
  void* du;
  void* ddelta;
  float* dA;
  float* dD;
  void* dz;
  float* ddelta_bias;
  float* dh0;
  const float* ckpt;  // [batch, dim, chunks, N]: state at each chunk start
  float* carry;       // [batch, dim, chunks, N]: Abar lambda entering each chunk from its end
  float* accB;        // [batch, N, L] float32 sums over channels
  float* accC;
  int64_t dim, dstate, seqlen, chunks;
  int softplus;
  int groups_per_block;  // channel groups of 16 per workgroup in the main pass
  // states n0 .. n0 + 15 in this launch of the main pass; with more than 16
  // states the launches run in order and carry the per-step sums over states
  // (ddelta before the softplus factor, du before D u, C . h) in psum
  int n0;
  int tile_mode;  // 0: the only tile, 1: first of several, 2: middle, 3: last
  float* psum;    // [3][batch * dim * seqlen] float32 partial sums (tile_mode 1..3)
};

// sum over the 16 lanes of a row; the row's last lane holds the total
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp0<kRowShr1>(v);
  v += dpp0<kRowShr2>(v);
  v += dpp0<kRowShr4>(v);
  v += dpp0<kRowShr8>(v);
  return v;
}


template <typename IO, int K, bool VEC, bool GATE, bool TILED>
__global__ void __launch_bounds__(256) scan_bwd_carry_kernel(const BwdArgs a) {
  constexpr int LPC = 16, CPB = 16, T = LPC * K, KP = K + 4, V = Io<IO>::V, TV = T / V;
  constexpr int NT = 16, NTH = 256, ITEMS = (NT * TV + NTH - 1) / NTH;
  __shared__ float4 sC4[NT * LPC * KP / 4];  // C rows of one 16-state tile
  __shared__ float sMu[CPB * kBwdMaxN], sA[CPB * kBwdMaxN];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int seg = lane % LPC;
  const int chb = wave * 4 + lane / LPC;
  const int64_t b = blockIdx.y, d0 = (int64_t)blockIdx.x * CPB, d = d0 + chb;
  const bool dvalid = d < a.dim;
  const int64_t N = a.dstate, L = a.seqlen;
  const int64_t row = (b * a.dim + (dvalid ? d : 0)) * L, bcrow = b * N * L;
  for (int i = threadIdx.x; i < CPB * N; i += NTH) {
    const int64_t c = i / N, n = i % N;
    const bool ok = d0 + c < a.dim;
    sMu[i] = (a.dfinal && ok) ? a.dfinal[(b * a.dim + d0 + c) * N + n] : 0.0f;
    sA[i] = ok ? a.A[(d0 + c) * N + n] : 0.0f;
  }
  // carries are kept per kCkptT-step block: the adjoint entering block k
  // from its end, Abar lambda at step (k + 1) kCkptT
  static_assert(T % kCkptT == 0 && kCkptT % K == 0, "carry blocks fall on lane starts");
  float* carry_ch = a.carry + (b * a.dim + d) * a.chunks * N;
  for (int64_t ci = (L + T - 1) / T - 1; ci >= 0; --ci) {
    const int64_t t0 = ci * T, tl = t0 + seg * K;
    Run<IO, K> rdy, rd, rz;
    run_load<IO, K, VEC>(rdy, a.dy, row, tl, L, dvalid);
    run_load<IO, K, VEC>(rd, a.delta, row, tl, L, dvalid);
    if constexpr (GATE) run_load<IO, K, VEC>(rz, a.z, row, tl, L, dvalid);
    __syncthreads();  // previous chunk's tile is no longer read; sMu/sA visible
    {
      const int64_t cend = ((t0 + T < L ? t0 + T : L) - 1) / kCkptT;  // last block of the chunk
      if constexpr (TILED) {
        if (dvalid)
          for (int64_t n = seg; n < N; n += LPC) carry_ch[cend * N + n] = sMu[chb * N + n];
      } else {
        if (dvalid && seg < N) carry_ch[cend * N + seg] = sMu[chb * N + seg];
      }
    }
    // C rows of states n0 .. n0 + nt - 1 -> LDS
    auto stage = [&](int64_t n0, int nt) {
#pragma unroll
      for (int k = 0; k < ITEMS; ++k) {
        const int item = threadIdx.x + k * NTH;
        if (item < nt * TV) {
          const int nl = item / TV, tloc = (item % TV) * V;
          Run<IO, V> rv;
          run_load<IO, V, VEC>(rv, a.Cm, bcrow + (n0 + nl) * L, t0 + tloc, L, true);
          float v[V];
          rv.unpack(v);
          float* dst = reinterpret_cast<float*>(sC4) + (nl * LPC + tloc / K) * KP + tloc % K;
#pragma unroll
          for (int q = 0; q < V; q += 4)
            *reinterpret_cast<float4*>(dst + q) = make_float4(v[q], v[q + 1], v[q + 2], v[q + 3]);
        }
      }
    };
    if constexpr (!TILED) {  // one tile: staged before the per-step values are formed
      stage(0, (int)N);
      __syncthreads();
    }
    float dl[K], dyc[K], S = 0.0f;
    {
      float raw[K], g[K], zz[K];
      rd.unpack(raw);
      rdy.unpack(g);
      if constexpr (GATE) rz.unpack(zz);
      const float bias = (a.delta_bias && dvalid) ? a.delta_bias[d] : 0.0f;
      step_log2<K>(raw, bias, a.softplus);
#pragma unroll
      for (int i = 0; i < K; ++i) {
        dl[i] = (tl + i < L) ? raw[i] : 0.0f;
        dyc[i] = GATE ? g[i] * silu_f(zz[i]) : g[i];
        S += dl[i];
      }
    }
    for (int64_t n0 = 0; n0 < N; n0 += NT) {
      const int nt = TILED ? (int)(N - n0 < NT ? N - n0 : NT) : (int)N;
      if constexpr (TILED) {
        if (n0 > 0) __syncthreads();  // every wave is done with the previous tile
        stage(n0, nt);
        __syncthreads();
      }
#pragma unroll 1
      for (int64_t n = n0; n < n0 + nt; ++n) {
        const float An = sA[chb * N + n];
        const float mu = sMu[chb * N + n];
        const float* pc = reinterpret_cast<const float*>(sC4) + ((n - n0) * LPC + seg) * KP;
        float av[K], gv[K];
#pragma unroll
        for (int i = 0; i < K; i += 4) {
          const float4 cc = *reinterpret_cast<const float4*>(pc + i);
          const float cq[4] = {cc.x, cc.y, cc.z, cc.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            av[i + q] = ex2(dl[i + q] * An);
            gv[i + q] = dyc[i + q] * cq[q];
          }
        }
        // fold the lane's steps backwards; the row's last lane starts from the
        // adjoint entering the chunk
        float Lam = gv[K - 1] + (seg == LPC - 1 ? mu : 0.0f);
#pragma unroll
        for (int i = K - 2; i >= 0; --i) Lam = fmaf(av[i + 1], Lam, gv[i]);
        float H = av[0] * Lam;
        row_scan16_rev(ex2(An * S), H);
        if (seg == 0) sMu[chb * N + n] = H;  // Abar lambda at the chunk's first step
        // lanes that start a block inside the chunk hand the block before it its carry
        if (seg > 0 && (seg * K) % kCkptT == 0 && tl < L && dvalid)
          carry_ch[(tl / kCkptT - 1) * N + n] = H;
      }
      if constexpr (!TILED) break;  // a single tile holds every state
    }
  }
}

// The carry pass for 16 states and bf16 rows, time-pipelined like the
// forward's scan_fwd_pipe_kernel: every lane runs the adjoint recurrence
// (the form above: lambda_t = dyc_t C_t + mu_{t+1}, mu_t = Abar_t lambda_t,
// backwards in t) over its own steps, with no fold and no scan.  Lane
// 16 r + c holds channel c and the states 4 j + r (items j = 0..3); the four
// waves are the 16-step segments of every 64-step chunk taken from the end
// (wave s runs steps 48 - 16 s .. 63 - 16 s), the chunks run from the last
// to the first, and mu passes from wave s to wave s + 1 (from wave 3 to wave
// 0 of the chunk before) through LDS slots with counted items, as in the
// forward.  Two chunks make a checkpoint block: mu at the first step of an
// even chunk is the carry of the block before it, and the last block's
// carry is the final-state gradient.  The per-step values (step size,
// dy silu(z)) of a lane's four steps of the next chunk are formed during
// this one and shared through LDS.
template <bool VEC, bool GATE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5)))
    scan_bwd_carry_pipe_kernel(const BwdArgs a) {
  using IO = uint16_t;
  constexpr int W = 4, K = 16, T = W * K, NS = 16, KP = K + 4;
  static_assert(kCkptT == 2 * T, "a checkpoint block is two chunks");
  __shared__ float4 sWave[W][NS * KP / 4];      // per wave: C rows of its segment
  __shared__ float4 sPrep[W][2 * 16 * KP / 4];  // per wave: step sizes, dy silu(z)
  __shared__ float sCarry[W][4][64];            // mu handed from wave s to s + 1
  __shared__ int sDone[W];
  __shared__ float sA[4][64];                   // A as [j][lane]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane >> 4, cl = lane & 15;
  const int64_t b = blockIdx.y;
  const int64_t d0 = (int64_t)blockIdx.x * 16;
  const int64_t d = d0 + cl;
  const bool dvalid = d < a.dim;
  const int64_t dc = dvalid ? d : d0;
  const int64_t L = a.seqlen;
  const int nchunks = (int)((L + T - 1) / T);  // L < 2^26 (launcher)
  const int64_t nblk = a.chunks;               // checkpoint blocks
  float* tile = reinterpret_cast<float*>(sWave[wave]);
  float* prep = reinterpret_cast<float*>(sPrep[wave]);
  const int seg0 = K * (W - 1 - wave);  // first step of this wave's segment in a chunk
  constexpr int ES = sizeof(IO);
  const int64_t seq_base = (b * a.dim + d0) * L;
  const int64_t nrows = a.dim - d0 < 16 ? a.dim - d0 : 16;
  const int seq_bytes = (int)(nrows * L * ES);
  const Rsrc dy_r = make_rsrc(static_cast<const IO*>(a.dy) + seq_base, seq_bytes);
  const Rsrc dl_r = make_rsrc(static_cast<const IO*>(a.delta) + seq_base, seq_bytes);
  const Rsrc z_r = make_rsrc(GATE ? static_cast<const IO*>(a.z) + seq_base : nullptr, GATE ? seq_bytes : 0);
  const Rsrc C_r = make_rsrc(static_cast<const IO*>(a.Cm) + b * NS * L, (int)(NS * L * ES));
  const int qstep = seg0 + 4 * r;  // first step of this lane's quad in a chunk
  // lane (r, c): its quad of channel c's rows and, for the C tile, of state c's row
  const uint32_t seq_off = (uint32_t)((cl * L + qstep) * ES);
  // carries: [channel][nblk][NS] rows from (b, d0) on
  const Rsrc cy_r = make_rsrc(a.carry + (b * a.dim + d0) * nblk * NS, (int)(nrows * nblk * NS * 4));
  const uint32_t cy_off = (uint32_t)(((dc - d0) * nblk * NS + r) * 4);

  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) sA[j][lane] = a.A[dc * NS + 4 * j + r];
  }
  const float bias = ((a.delta_bias && dvalid) ? a.delta_bias[d] : 0.0f) * kLog2e;  // bias / ln 2

  // The chunk body comes in two forms: FULL for whole chunks (every chunk
  // but the last, and the last when 64 divides L), whose steps need no lane
  // masks, and the general one.  The look-ahead loads are of whole chunks
  // and are issued unmasked in every chunk (in the last chunks processed,
  // the sequence's first, they read chunk 0 again: in bounds, unused), so
  // that the number of memory operations
  // after each load is the same on every path and the wait for a load does
  // not have to drain the younger ones.
  auto left = [&](int c) { return (int)(L - (int64_t)c * T < T ? L - (int64_t)c * T : T); };
  auto coff = [&](int c) { return (uint32_t)c * (uint32_t)(T * ES); };
  auto quad_n = [&](int c, auto full) { return decltype(full)::value ? 4 : left(c) - qstep; };
  struct Raw {
    Quad dy, dl, z;
  };
  auto load_raw = [&](Raw& q, int c, auto full) {
    const int n = quad_n(c, full);
    quad_load<VEC>(q.dy, dy_r, seq_off, coff(c), n);
    quad_load<VEC>(q.dl, dl_r, seq_off, coff(c), n);
    if constexpr (GATE) quad_load<VEC>(q.z, z_r, seq_off, coff(c), n);
  };
  Quad cq_raw;
  auto load_c = [&](int c, auto full) { quad_load<VEC>(cq_raw, C_r, seq_off, coff(c), quad_n(c, full)); };
  // steps i, i + 1 of the lane's quad of chunk c -> LDS: the step size in
  // log2 units (dl = delta / ln 2 from the raw step by one fma, so that Abar
  // = exp2(dl A); zero past L, an identity step) and dy silu(z)
  auto prep_pair = [&](const Raw& q, int i, int c, auto full) {
    float v[2], g[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float xl = fmaf(q.dl.at(i + k), kLog2e, bias);  // (raw + bias) / ln 2
      float s = a.softplus ? softplus_xl(xl) : xl;
      if constexpr (!decltype(full)::value) s = qstep + i + k < left(c) ? s : 0.0f;
      v[k] = s;
      g[k] = GATE ? q.dy.at(i + k) * silu_f(q.z.at(i + k)) : q.dy.at(i + k);
    }
    *reinterpret_cast<float2*>(prep + cl * KP + 4 * r + i) = make_float2(v[0], v[1]);
    *reinterpret_cast<float2*>(prep + 16 * KP + cl * KP + 4 * r + i) = make_float2(g[0], g[1]);
  };

  const std::false_type general{};
  const int clast = nchunks - 1;
  Raw nxt{};
  {
    Raw first;
    load_raw(first, clast, general);
    load_c(clast, general);
    load_raw(nxt, clast > 0 ? clast - 1 : 0, std::true_type{});
    prep_pair(first, 0, clast, general);
    prep_pair(first, 2, clast, general);
  }
  if (wave == W - 1) {
    // mu entering the last step is the final-state gradient; it is also the
    // last block's carry
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float mu = (a.dfinal && dvalid) ? a.dfinal[(b * a.dim + d) * NS + 4 * j + r] : 0.0f;
      sCarry[W - 1][j][lane] = mu;
      if (dvalid) buf_st32(__float_as_uint(mu), cy_r, cy_off, (uint32_t)(((nblk - 1) * NS + 4 * j) * 4));
    }
  }
  if (threadIdx.x < W) sDone[threadIdx.x] = 0;
  __syncthreads();
  const int pred = (wave + W - 1) & (W - 1);

  // chunk c, the p-th processed
  auto chunk = [&](const int c, const int p, auto full) {
    {
      opaque(cq_raw);
      *reinterpret_cast<float4*>(tile + cl * KP + 4 * r) =
          make_float4(cq_raw.at(0), cq_raw.at(1), cq_raw.at(2), cq_raw.at(3));
    }
    load_c(c > 0 ? c - 1 : 0, std::true_type{});
    wave_lds_sync();
    float dl[K], g[K];
#pragma unroll
    for (int i = 0; i < K; i += 4) {
      const float4 pv = *reinterpret_cast<const float4*>(prep + cl * KP + i);
      const float4 qv = *reinterpret_cast<const float4*>(prep + 16 * KP + cl * KP + i);
      dl[i] = pv.x; dl[i + 1] = pv.y; dl[i + 2] = pv.z; dl[i + 3] = pv.w;
      g[i] = qv.x; g[i + 1] = qv.y; g[i + 2] = qv.z; g[i + 3] = qv.w;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int item = 4 * p + j;
      // the predecessor's hand-over of this item (bounded wait, as in the
      // forward; in the first chunk wave 0 needs none: its slots hold dfinal)
      {
        const int need = wave == 0 ? item - 3 : item + 1;
#pragma unroll 1
        for (int spin = 0; spin < (1 << 23); ++spin) {
          if (__builtin_amdgcn_readfirstlane(__hip_atomic_load(&sDone[pred], __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_WORKGROUP)) >= need)
            break;
          __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      }
      float mu = sCarry[pred][j][lane];
      const float A = sA[j][lane];
      const float* pc = tile + (4 * j + r) * KP;
#pragma unroll
      for (int i = K - 4; i >= 0; i -= 4) {
        const float4 cc = *reinterpret_cast<const float4*>(pc + i);
        const float cq[4] = {cc.x, cc.y, cc.z, cc.w};
#pragma unroll
        for (int q = 3; q >= 0; --q) {
          const float lam = fmaf(g[i + q], cq[q], mu);
          mu = ex2(dl[i + q] * A) * lam;
        }
      }
      sCarry[wave][j][lane] = mu;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      if (lane == 0) __hip_atomic_store(&sDone[wave], item + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      // mu at the first step of an even chunk c >= 2: the carry of block c / 2 - 1
      if (wave == W - 1 && (c & 1) == 0 && c >= 2 && dvalid)
        buf_st32(__float_as_uint(mu), cy_r, cy_off, (uint32_t)(((c / 2 - 1) * NS + 4 * j) * 4));
      if (j == 1 || j == 2) {
        if (j == 1) {
          opaque(nxt.dy);
          opaque(nxt.dl);
          if constexpr (GATE) opaque(nxt.z);
        }
        if (c >= 1) prep_pair(nxt, 2 * (j - 1), c - 1, std::true_type{});  // chunk c - 1 is whole
      }
      if (j == 3) load_raw(nxt, c > 1 ? c - 2 : 0, std::true_type{});
    }
  };
  if (L % T == 0) chunk(clast, 0, std::true_type{});
  else chunk(clast, 0, general);
  for (int c = clast - 1, p = 1; c >= 0; --c, ++p) chunk(c, p, std::true_type{});
}

// Two consecutive elements starting at an even index (4- or 8-byte aligned).
template <typename IO>
struct Pair;
template <>
struct Pair<float> {
  float2 v;
  __device__ void load(const void* p, int64_t i) { v = *reinterpret_cast<const float2*>(static_cast<const float*>(p) + i); }
  __device__ float get(int k) const { return k ? v.y : v.x; }
};
template <>
struct Pair<uint16_t> {
  uint32_t v;
  __device__ void load(const void* p, int64_t i) { v = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + i); }
  __device__ float get(int k) const { return k ? bf_hi(v) : bf_lo(v); }
};

template <typename IO, int K, bool VEC, bool ZOH, bool GATE, bool TILED>
// two waves per SIMD: the register file holds two of these waves only if
// every instantiation stays within 256 registers (AGPRs included)
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
scan_bwd_main_kernel(const BwdArgs a) {
  static_assert(K == 8, "the channel reduction of dB and dC handles eight steps per lane");
  constexpr int LPC = 16, T = LPC * K, KP = K + 4, V = Io<IO>::V, TV = T / V;
  constexpr int NT = 16, NTH = 256, ITEMS = (2 * NT * TV + NTH - 1) / NTH;
  constexpr int CPG = 4;  // channels per group: one per 16-lane row
  constexpr int NW = 4;   // waves sharing a group
  // Work split inside a group: wave w runs the recurrences for states
  // w, w + 4, w + 8, w + 12 over all steps, and the per-step work (step
  // size, gate, output gradients) for steps 2w and 2w + 1 of every lane.
  __shared__ float4 sB4[NT * LPC * KP / 4];
  __shared__ float4 sC4[NT * LPC * KP / 4];
  constexpr int SP = K + 4;  // padded per-lane row: 16-byte reads of a wave hit distinct banks
  __shared__ float4 sRed4[NW * 3 * 64 * SP / 4];  // [wave][ddt, du, yc][lane][step] partial sums
  __shared__ float4 sPrep4[3 * 64 * SP / 4];      // [delta, u, dy silu(z)][lane][step]
  __shared__ float sPar[NW * 3 * CPG * NT];      // per wave: A, state at chunk start, carry
  // a group's per-channel sums, double-buffered by group parity: dA of the
  // group's 4 channels x 16 states, and each wave's part of ddelta_bias and dD
  __shared__ float sGdA[2][CPG][NT];
  __shared__ float sGbD[2][2][NW][CPG];
  float* sRed = reinterpret_cast<float*>(sRed4);
  float* sPrep = reinterpret_cast<float*>(sPrep4);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int seg = lane % LPC, row = lane / LPC;
  const bool first = seg == 0, last = seg == LPC - 1;
  const int red_row = red_step(row);
  const int64_t b = blockIdx.z, ci = blockIdx.y;
  const int64_t N = a.dstate, L = a.seqlen;
  const int n0 = TILED ? a.n0 : 0;  // this launch's states: n0 .. n0 + nt - 1
  const int nt = TILED ? (int)(N - n0 < NT ? N - n0 : NT) : (int)N;
  const int64_t t0 = ci * T, tl = t0 + seg * K, bcrow = b * N * L;
  const int s0 = 2 * wave;               // this wave's two steps
  const int64_t ts = tl + s0;            // their time index
  const bool ok0 = ts < L, ok1 = ts + 1 < L;
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    const int item = threadIdx.x + k * NTH;
    if (item < 2 * nt * TV) {
      const int tensor = item / (nt * TV);
      const int r = item % (nt * TV);
      const int nl = r / TV, tloc = (r % TV) * V;
      Run<IO, V> rv;
      run_load<IO, V, VEC>(rv, tensor ? a.Cm : a.Bm, bcrow + (n0 + nl) * L, t0 + tloc, L, true);
      float v[V];
      rv.unpack(v);
      float* dst = reinterpret_cast<float*>(tensor ? sC4 : sB4) + (nl * LPC + tloc / K) * KP + tloc % K;
#pragma unroll
      for (int q = 0; q < V; q += 4)
        *reinterpret_cast<float4*>(dst + q) = make_float4(v[q], v[q + 1], v[q + 2], v[q + 3]);
    }
  }

  // dB and dC of this chunk for states wave + 4j and the lane's K steps,
  // summed over every channel of the lane's row the workgroup visits; the sum
  // over the wave's four rows is taken once, at the end
  float accB[4][K], accC[4][K];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int q = 0; q < K; ++q) accB[j][q] = accC[j][q] = 0.0f;

  const int64_t ngroups = (a.dim + CPG - 1) / CPG;
  const int64_t g_begin = (int64_t)blockIdx.x * a.groups_per_block;
  const int64_t g_end = min(g_begin + a.groups_per_block, ngroups);
  float* par = sPar + wave * 3 * CPG * NT;
  // loads of group g + 1 are issued while group g computes
  Pair<IO> nu, nd, ndy, nz;
  float npar[3], nbias = 0.0f, nDd = 0.0f;
  float2 nps[3] = {};  // partial sums of earlier tiles at this wave's two steps
  auto fetch = [&](int64_t g) {
    const int64_t d = g * CPG + row;
    const bool okd = d < a.dim;
    const int64_t ch = b * a.dim + (okd ? d : 0);
    // the pair is read whole when it starts inside the row (L is even on
    // the vectorised path); otherwise element by element
    const int64_t base = ch * L + ts;
    if (okd && VEC && ok1) {
      nu.load(a.u, base);
      nd.load(a.delta, base);
      ndy.load(a.dy, base);
      if constexpr (GATE) nz.load(a.z, base);
    } else {
      float e[4][2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const bool okk = okd && ts + k < L;
        e[0][k] = okk ? Io<IO>::ld1(a.u, base + k) : 0.0f;
        e[1][k] = okk ? Io<IO>::ld1(a.delta, base + k) : 0.0f;
        e[2][k] = okk ? Io<IO>::ld1(a.dy, base + k) : 0.0f;
        e[3][k] = (GATE && okk) ? Io<IO>::ld1(a.z, base + k) : 0.0f;
      }
      if constexpr (std::is_same<IO, float>::value) {
        nu.v = make_float2(e[0][0], e[0][1]); nd.v = make_float2(e[1][0], e[1][1]);
        ndy.v = make_float2(e[2][0], e[2][1]); nz.v = make_float2(e[3][0], e[3][1]);
      } else {
        nu.v = pack_bf16x2(e[0][0], e[0][1]); nd.v = pack_bf16x2(e[1][0], e[1][1]);
        ndy.v = pack_bf16x2(e[2][0], e[2][1]); nz.v = pack_bf16x2(e[3][0], e[3][1]);
      }
    }
    const int64_t cb = (ch * a.chunks + ci) * N + n0 + seg;
    const bool own = okd && seg < nt;
    npar[0] = own ? a.A[(okd ? d : 0) * N + n0 + seg] : 0.0f;
    npar[1] = own ? a.ckpt[cb] : 0.0f;
    npar[2] = own ? a.carry[cb] : 0.0f;
    nbias = (a.delta_bias && okd) ? a.delta_bias[d] : 0.0f;
    nDd = (a.Dskip && okd) ? a.Dskip[d] : 0.0f;
    if constexpr (TILED) {
      if (a.tile_mode >= 2) {
        const int64_t bdl = a.dim * L * (int64_t)gridDim.z;  // batch * dim * seqlen
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          nps[q].x = (okd && ok0) ? a.psum[q * bdl + base] : 0.0f;
          nps[q].y = (okd && ok1) ? a.psum[q * bdl + base + 1] : 0.0f;
        }
      }
    }
  };
  // Outputs of group g are written at the top of group g + 1, next to the
  // loads of group g + 2: a wait for those loads then finds the writes long
  // done instead of stalling on writes just issued.
  float p_du[2] = {0.0f, 0.0f}, p_dr[2] = {0.0f, 0.0f}, p_dz[2] = {0.0f, 0.0f};
  float p_db = 0.0f, p_dD = 0.0f;
  int64_t p_d = -1;  // channel of the pending outputs (-1: none)
  // partial tiles (tile_mode 1, 2) leave their per-step sums in psum instead
  const bool partial = TILED && (a.tile_mode == 1 || a.tile_mode == 2);
  auto flush = [&]() {
    if (p_d < 0 || p_d >= a.dim) return;
    const int64_t pch = b * a.dim + p_d;
    const int64_t base = pch * L + ts;
    if (partial) {
      const int64_t bdl = a.dim * L * (int64_t)gridDim.z;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (k ? ok1 : ok0) {
          a.psum[base + k] = p_dr[k];
          a.psum[bdl + base + k] = p_du[k];
          a.psum[2 * bdl + base + k] = p_dz[k];
        }
      }
    } else if (VEC && ok1) {
      if constexpr (std::is_same<IO, float>::value) {
        *reinterpret_cast<float2*>(static_cast<float*>(a.du) + base) = make_float2(p_du[0], p_du[1]);
        *reinterpret_cast<float2*>(static_cast<float*>(a.ddelta) + base) = make_float2(p_dr[0], p_dr[1]);
        if constexpr (GATE)
          *reinterpret_cast<float2*>(static_cast<float*>(a.dz) + base) = make_float2(p_dz[0], p_dz[1]);
      } else {
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.du) + base) = pack_bf16x2(p_du[0], p_du[1]);
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.ddelta) + base) = pack_bf16x2(p_dr[0], p_dr[1]);
        if constexpr (GATE)
          *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.dz) + base) = pack_bf16x2(p_dz[0], p_dz[1]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (k ? ok1 : ok0) {
          Io<IO>::st1(a.du, base + k, p_du[k]);
          Io<IO>::st1(a.ddelta, base + k, p_dr[k]);
          if constexpr (GATE) Io<IO>::st1(a.dz, base + k, p_dz[k]);
        }
      }
    }
  };
  // The per-channel sums of group gp (dA, ddelta_bias, dD), gathered in LDS
  // buffer bp, go out as contiguous runs of atomic adds: wave w adds channel
  // w's dA over the tile's states; waves 0 and 1 add the group's four
  // ddelta_bias and four dD, each summed over the four waves' parts.  (One
  // atomic per lane and state, scattered over the channels, counted 32 bytes
  // of memory writes each.)
  auto issue_sums = [&](int64_t gp, int bp) {
    const int64_t dp = gp * CPG + wave;
    if (dp < a.dim && lane < nt) unsafeAtomicAdd(&a.dA[dp * N + n0 + lane], sGdA[bp][wave][lane]);
    if (!partial && wave < 2 && lane < CPG) {
      const int64_t dc = gp * CPG + lane;
      float* dst = wave ? a.dD : a.ddelta_bias;
      if (dst && dc < a.dim) {
        float v = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) v += sGbD[bp][wave][ww][lane];
        unsafeAtomicAdd(&dst[dc], v);
      }
    }
  };
  if (g_begin < g_end) fetch(g_begin);
  for (int64_t g = g_begin; g < g_end; ++g) {
    const int64_t d = g * CPG + row;
    const bool dvalid = d < a.dim;
    const int64_t ch = b * a.dim + (dvalid ? d : 0);
    const Pair<IO> pu = nu, pd = nd, pdy = ndy, pz = nz;
    const float bias = nbias, Dd = nDd;
    float2 ps[3];
    if constexpr (TILED) {
      ps[0] = nps[0]; ps[1] = nps[1]; ps[2] = nps[2];
    }
    par[row * NT + seg] = npar[0];
    par[(CPG + row) * NT + seg] = npar[1];
    par[(2 * CPG + row) * NT + seg] = npar[2];
    if (g + 1 < g_end) fetch(g + 1);
    flush();
    // ---- per-step inputs of this wave's two steps, shared through LDS
    float xs[2], us[2], gs[2], zs[2], dycs[2];
    {
      float2 dtp, dyp;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        xs[k] = pd.get(k) + bias;
        us[k] = pu.get(k);
        gs[k] = pdy.get(k);
        zs[k] = GATE ? pz.get(k) : 0.0f;
        const float v = a.softplus ? softplus_log2(xs[k]) : xs[k] * kLog2e;
        const float dtk = (k ? ok1 : ok0) ? v * kLn2 : 0.0f;
        dycs[k] = GATE ? gs[k] * silu_f(zs[k]) : gs[k];
        if (k) { dtp.y = dtk; dyp.y = dycs[k]; } else { dtp.x = dtk; dyp.x = dycs[k]; }
      }
      *reinterpret_cast<float2*>(sPrep + (0 * 64 + lane) * SP + s0) = dtp;
      *reinterpret_cast<float2*>(sPrep + (1 * 64 + lane) * SP + s0) = make_float2(us[0], us[1]);
      *reinterpret_cast<float2*>(sPrep + (2 * 64 + lane) * SP + s0) = dyp;
    }
    __syncthreads();  // every wave's steps are in; the previous group's sums are read
    if (g > g_begin) issue_sums(g - 1, (int)((g - 1) & 1));
    const int gbuf = (int)(g & 1);
    // lb[i] (delta*B rule): sum over this wave's states of lambda_t B_t, from
    // which du and the input's part of ddelta follow once per step
    float dt[K], uu[K], w[K], dyc[K], yc[K], ddt[K], du[K], lb[K];
    float S = 0.0f;  // sum of the lane's steps, in log2 units
#pragma unroll
    for (int i = 0; i < K; i += 4) {
      const float4 q0 = *reinterpret_cast<const float4*>(sPrep + (0 * 64 + lane) * SP + i);
      const float4 q1 = *reinterpret_cast<const float4*>(sPrep + (1 * 64 + lane) * SP + i);
      const float4 q2 = *reinterpret_cast<const float4*>(sPrep + (2 * 64 + lane) * SP + i);
      dt[i] = q0.x; dt[i + 1] = q0.y; dt[i + 2] = q0.z; dt[i + 3] = q0.w;
      uu[i] = q1.x; uu[i + 1] = q1.y; uu[i + 2] = q1.z; uu[i + 3] = q1.w;
      dyc[i] = q2.x; dyc[i + 1] = q2.y; dyc[i + 2] = q2.z; dyc[i + 3] = q2.w;
    }
#pragma unroll
    for (int i = 0; i < K; ++i) {
      S += dt[i];
      w[i] = dt[i] * uu[i];
      yc[i] = 0.0f;
      ddt[i] = 0.0f;
      du[i] = 0.0f;
      lb[i] = 0.0f;
    }
    S *= kLog2e;
    const float* pA = par + row * NT;
    const float* pH = par + (CPG + row) * NT;
    const float* pM = par + (2 * CPG + row) * NT;
    // the four states' parameters, read once ahead of the state loop (rows
    // past N read another row's values, which no state then uses); the ZOH
    // instantiation has no registers to spare for them and reads each in turn
    float Av[4], Hv[4], Mv[4];
    if constexpr (!ZOH) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Av[j] = pA[wave + NW * j];
        Hv[j] = pH[wave + NW * j];
        Mv[j] = pM[wave + NW * j];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = wave + NW * j;
      if (n < nt) {
        const float An = ZOH ? pA[n] : Av[j];
        const float hs = ZOH ? pH[n] : Hv[j];      // state before the chunk
        const float mu_end = ZOH ? pM[n] : Mv[j];  // Abar lambda entering from the chunk's end
        const float Anl = An * kLog2e;
        const float* pb = reinterpret_cast<const float*>(sB4) + (n * LPC + seg) * KP;
        const float* pc = reinterpret_cast<const float*>(sC4) + (n * LPC + seg) * KP;
        float av[K], xv[K], cf[K], hh[K + 1], bq[K], cq[K];
#pragma unroll
        for (int i = 0; i < K; i += 4) {
          const float4 bb = *reinterpret_cast<const float4*>(pb + i);
          const float4 cc = *reinterpret_cast<const float4*>(pc + i);
          bq[i] = bb.x; bq[i + 1] = bb.y; bq[i + 2] = bb.z; bq[i + 3] = bb.w;
          cq[i] = cc.x; cq[i + 1] = cc.y; cq[i + 2] = cc.z; cq[i + 3] = cc.w;
        }
#pragma unroll
        for (int i = 0; i < K; ++i) {
          av[i] = ex2(dt[i] * Anl);
          if constexpr (ZOH) {
            cf[i] = An != 0.0f ? expm1_f(dt[i] * An, av[i]) * rcp(An) : dt[i];
            xv[i] = cf[i] * uu[i] * bq[i];
          } else {
            xv[i] = w[i] * bq[i];
          }
        }
        // ---- forward: the states of the chunk, from the checkpoint
        const float Al = ex2(An * S);
        float H = fmaf(av[0], first ? hs : 0.0f, xv[0]);
#pragma unroll
        for (int i = 1; i < K; ++i) H = fmaf(av[i], H, xv[i]);
        row_scan16(Al, H);
        const float He = dpp0<kRowShr1>(H);
        hh[0] = first ? hs : He;
#pragma unroll
        for (int i = 0; i < K; ++i) {
          hh[i + 1] = fmaf(av[i], hh[i], xv[i]);
          if constexpr (GATE) yc[i] = fmaf(cq[i], hh[i + 1], yc[i]);
        }
        // ---- adjoint: backwards over the chunk from the stored carry
        float Lam = fmaf(dyc[K - 1], cq[K - 1], last ? mu_end : 0.0f);
#pragma unroll
        for (int i = K - 2; i >= 0; --i) Lam = fmaf(av[i + 1], Lam, dyc[i] * cq[i]);
        float H2 = av[0] * Lam;
        row_scan16_rev(Al, H2);
        const float Hn = dpp0<kRowShl1>(H2);
        float mu = last ? mu_end : Hn;
        float dAacc = 0.0f;
#pragma unroll
        for (int i = K - 1; i >= 0; --i) {
          const float lam = fmaf(dyc[i], cq[i], mu);  // lambda_t
          const float mun = av[i] * lam;               // Abar_t lambda_t
          const float daa = mun * hh[i];               // lambda_t Abar_t h_{t-1}
          ddt[i] = fmaf(daa, An, ddt[i]);
          dAacc = fmaf(daa, dt[i], dAacc);
          if constexpr (ZOH) {
            const float lbn = lam * bq[i];
            const float dbeta = lbn * uu[i];  // lambda B u
            ddt[i] = fmaf(dbeta, av[i], ddt[i]);
            // d cf / dA = (dt Abar - cf) / A, or where |dt A| < 1/32 (and that
            // difference would cancel) its series dt^2 (1/2 + r/3 + r^2/8 + r^3/30)
            const float r = dt[i] * An;
            const float dcf = fabsf(r) < 0.03125f
                                  ? dt[i] * dt[i] * fmaf(r, fmaf(r, fmaf(r, 1.0f / 30, 0.125f), 1.0f / 3), 0.5f)
                                  : (dt[i] * av[i] - cf[i]) * rcp(An);
            dAacc = fmaf(dbeta, dcf, dAacc);
            accB[j][i] = fmaf(lam, cf[i] * uu[i], accB[j][i]);
            du[i] = fmaf(lbn, cf[i], du[i]);
          } else {
            lb[i] = fmaf(lam, bq[i], lb[i]);
            accB[j][i] = fmaf(lam, w[i], accB[j][i]);
          }
          accC[j][i] = fmaf(dyc[i], hh[i + 1], accC[j][i]);
          mu = mun;
        }
        dAacc = row_sum16(dAacc);
        if (last) sGdA[gbuf][row][n] = dAacc;
        if (ci == 0 && first && dvalid && a.dh0) a.dh0[ch * N + n0 + n] = mu;
      }
    }
    if constexpr (!ZOH) {
#pragma unroll
      for (int i = 0; i < K; ++i) {
        ddt[i] = fmaf(lb[i], uu[i], ddt[i]);
        du[i] = lb[i] * dt[i];
      }
    }
    // ---- per-step gradients: sum the four waves' partials for this wave's
    // two steps
    {
      float* red = sRed + wave * 3 * 64 * SP;
#pragma unroll
      for (int i = 0; i < K; i += 4) {
        *reinterpret_cast<float4*>(red + (0 * 64 + lane) * SP + i) = make_float4(ddt[i], ddt[i + 1], ddt[i + 2], ddt[i + 3]);
        *reinterpret_cast<float4*>(red + (1 * 64 + lane) * SP + i) = make_float4(du[i], du[i + 1], du[i + 2], du[i + 3]);
        if constexpr (GATE)
          *reinterpret_cast<float4*>(red + (2 * 64 + lane) * SP + i) = make_float4(yc[i], yc[i + 1], yc[i + 2], yc[i + 3]);
      }
    }
    __syncthreads();
    {
      float2 sddt = make_float2(0.0f, 0.0f), sdu = sddt, syc = sddt;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float* rr = sRed + ww * 3 * 64 * SP + lane * SP + s0;
        const float2 p0 = *reinterpret_cast<const float2*>(rr);
        const float2 p1 = *reinterpret_cast<const float2*>(rr + 64 * SP);
        sddt.x += p0.x; sddt.y += p0.y;
        sdu.x += p1.x; sdu.y += p1.y;
        if constexpr (GATE) {
          const float2 p2 = *reinterpret_cast<const float2*>(rr + 2 * 64 * SP);
          syc.x += p2.x; syc.y += p2.y;
        }
      }
      if constexpr (TILED) {
        if (a.tile_mode >= 2) {
          sddt.x += ps[0].x; sddt.y += ps[0].y;
          sdu.x += ps[1].x; sdu.y += ps[1].y;
          syc.x += ps[2].x; syc.y += ps[2].y;
        }
      }
      float dbacc = 0.0f, dDacc = 0.0f;
      if (partial) {
        p_dr[0] = sddt.x; p_dr[1] = sddt.y;
        p_du[0] = sdu.x; p_du[1] = sdu.y;
        p_dz[0] = syc.x; p_dz[1] = syc.y;
      } else {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const bool okk = k ? ok1 : ok0;
          const float s_ddt = k ? sddt.y : sddt.x, s_du = k ? sdu.y : sdu.x, s_yc = k ? syc.y : syc.x;
          const float sig = a.softplus ? rcp(1.0f + ex2(-xs[k] * kLog2e)) : 1.0f;
          p_dr[k] = okk ? s_ddt * sig : 0.0f;
          dbacc += p_dr[k];
          dDacc += okk ? dycs[k] * us[k] : 0.0f;
          p_du[k] = fmaf(dycs[k], Dd, s_du);
          if constexpr (GATE) {
            const float sz = rcp(1.0f + ex2(-zs[k] * kLog2e));
            p_dz[k] = gs[k] * fmaf(Dd, us[k], s_yc) * sz * fmaf(zs[k], 1.0f - sz, 1.0f);
          }
        }
      }
      p_db = row_sum16(dbacc);
      p_dD = row_sum16(dDacc);
      if (last) {
        sGbD[gbuf][0][wave][row] = p_db;
        sGbD[gbuf][1][wave][row] = p_dD;
      }
      p_d = d;
    }
  }
  flush();
  __syncthreads();  // the last group's sums are in LDS
  if (g_begin < g_end) issue_sums(g_end - 1, (int)((g_end - 1) & 1));
  // ---- this chunk's dB and dC from every channel the block visited.
  // After the row sums, lane (seg, row) holds steps seg K + red_row (lo) and
  // seg K + red_row + 4 (hi).  The hi values are rotated by half a row
  // (segments seg and seg +- 8 trade them), so that the first atomic of each
  // tensor covers segments 0..7 and the second segments 8..15, each as whole
  // 32-byte runs of eight steps (two atomics per sector otherwise).
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = wave + NW * j;
    if (n < nt) {
      float* pBn = a.accB + (b * N + n0 + n) * L;
      float* pCn = a.accC + (b * N + n0 + n) * L;
      float bl, bh, cl, chh;
      rows_sum8(accB[j], bl, bh);
      rows_sum8(accC[j], cl, chh);
      const float bh8 = dpp<0x128, 0xf>(0.0f, bh);   // row_ror:8: segment seg -+ 8's hi
      const float ch8 = dpp<0x128, 0xf>(0.0f, chh);
      const bool low = seg < 8;
      // first atomic: segments 0..7; second: segments 8..15
      const int64_t ta = t0 + (low ? seg * K + red_row : (seg - 8) * K + red_row + 4);
      const int64_t tb = t0 + (low ? (seg + 8) * K + red_row + 4 : seg * K + red_row);
      if (ta < L) {
        unsafeAtomicAdd(pBn + ta, low ? bl : bh8);
        unsafeAtomicAdd(pCn + ta, low ? cl : ch8);
      }
      if (tb < L) {
        unsafeAtomicAdd(pBn + tb, low ? bh8 : bl);
        unsafeAtomicAdd(pCn + tb, low ? ch8 : cl);
      }
    }
  }
}

__global__ void __launch_bounds__(256) fill_zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0.0f;
}

template <typename IO>
__global__ void __launch_bounds__(256) store_io_kernel(const float* src, void* dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    Io<IO>::st1(dst, i, src[i]);
}

// ---------------------------------------------------------------- causal conv1d
//
// Depthwise causal convolution of width W with an optional silu, the step in
// front of the scan in the Mamba block ("State-space models", section
// "Mamba: selection"): pre_t = bias + sum_k w_k x_{t-(W-1)+k} on a sequence
// padded on the left (by zeros or a carried state of the W-1 previous
// inputs), out_t = silu(pre_t).  HBM-bound: one read of x and one write of
// out.  A thread owns one 16-byte vector of V consecutive steps of a row; the
// W-1 inputs before its vector come from the neighbouring lane by a DPP
// wave shift, the first lane of each wave loads them itself.

#ifndef SELSCAN_CONV_BWD_VPW
#define SELSCAN_CONV_BWD_VPW 4  // spans of 256 runs per workgroup in the conv1d backward
#endif

struct ConvArgs {
  const void* x;
  const float* w;       // [dim, W]
  const float* bias;    // [dim] or null
  const float* state_in;  // [batch, dim, W-1] or null (zeros)
  void* out;
  const void* dout;     // backward
  void* dx;
  float* dw;
  float* dbias;
  float* dstate_in;
  int64_t rows, dim, seqlen;
  int silu;
};

template <int CTRL>
__device__ __forceinline__ float wave_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kWaveShl1 = 0x130;

// x of row r at step t, t in [-(W-1), L): the carried state before t = 0.
template <typename IO, int W>
__device__ __forceinline__ float conv_x_at(const ConvArgs& a, int64_t r, int64_t t) {
  if (t >= 0) return t < a.seqlen ? Io<IO>::ld1(a.x, r * a.seqlen + t) : 0.0f;
  return a.state_in ? a.state_in[r * (W - 1) + (W - 1) + t] : 0.0f;
}

// the V steps of this thread (zero past L)
template <typename IO, bool VEC>
__device__ __forceinline__ void conv_load_run(const void* p, int64_t base, int64_t t0, int64_t L,
                                              float* v) {
  constexpr int V = Io<IO>::V;
  if (VEC && t0 + V <= L) {
    Io<IO>::ldv(p, base + t0, v);
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = t0 + i < L ? Io<IO>::ld1(p, base + t0 + i) : 0.0f;
  }
}

template <typename IO, bool VEC>
__device__ __forceinline__ void conv_store_run(void* p, int64_t base, int64_t t0, int64_t L,
                                               const float* v) {
  constexpr int V = Io<IO>::V;
  if (VEC && t0 + V <= L) {
    Io<IO>::stv(p, base + t0, v);
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (t0 + i < L) Io<IO>::st1(p, base + t0 + i, v[i]);
  }
}

// Loads of one thread's run and of the wave's halo, issued without waiting:
// addresses are clamped into bounds and out-of-range values are replaced
// only after the loads (a branch around a load would wait for it at once).
template <typename IO, int W, bool VEC>
struct ConvRun {
  static constexpr int V = Io<IO>::V, H = W - 1;
  using Raw = typename std::conditional<std::is_same<IO, float>::value, float4, uint4>::type;
  Raw raw;
  float hx[H > 0 ? H : 1], hs[H > 0 ? H : 1];
  __device__ void load(const ConvArgs& a, const void* p, int64_t r, int64_t base, int64_t t0,
                       bool first_lane, bool want_halo) {
    const int64_t L = a.seqlen;
    if constexpr (VEC) {
      const int64_t tc = t0 < L ? t0 : L - V;  // L is a multiple of V here
      raw = *reinterpret_cast<const Raw*>(static_cast<const IO*>(p) + base + tc);
    }
    if (want_halo && first_lane) {
#pragma unroll
      for (int j = 0; j < H; ++j) {
        const int64_t t = t0 - H + j;
        hx[j] = Io<IO>::ld1(p, base + (t > 0 ? t : 0));
        const int64_t si = H + t < 0 ? 0 : (H + t > H - 1 ? H - 1 : H + t);
        hs[j] = a.state_in ? a.state_in[r * H + si] : 0.0f;
      }
    }
  }
  // the run's V values, zero past L
  __device__ void values(const void* p, int64_t base, int64_t t0, int64_t L, float* v) const {
    if constexpr (VEC) {
      float u[V];
      if constexpr (std::is_same<IO, float>::value) {
        u[0] = raw.x; u[1] = raw.y; u[2] = raw.z; u[3] = raw.w;
      } else {
        u[0] = bf_lo(raw.x); u[1] = bf_hi(raw.x); u[2] = bf_lo(raw.y); u[3] = bf_hi(raw.y);
        u[4] = bf_lo(raw.z); u[5] = bf_hi(raw.z); u[6] = bf_lo(raw.w); u[7] = bf_hi(raw.w);
      }
#pragma unroll
      for (int i = 0; i < V; ++i) v[i] = t0 < L ? u[i] : 0.0f;
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) v[i] = t0 + i < L ? Io<IO>::ld1(p, base + t0 + i) : 0.0f;
    }
  }
  // input before the run at position j of the halo (first lane of a wave)
  __device__ float halo(int64_t t0, int j) const { return t0 - H + j >= 0 ? hx[j] : hs[j]; }
};

template <typename IO, int W, bool VEC>
__global__ void __launch_bounds__(256) conv1d_fwd_kernel(const ConvArgs a) {
  constexpr int V = Io<IO>::V, H = W - 1;
  const int lane = threadIdx.x & 63;
  const int64_t L = a.seqlen;
  const int64_t t0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;
  for (int64_t r = blockIdx.y; r < a.rows; r += gridDim.y) {
    const int64_t d = r % a.dim, base = r * L;
    float wk[W];
#pragma unroll
    for (int k = 0; k < W; ++k) wk[k] = a.w[d * W + k];
    const float b = a.bias ? a.bias[d] : 0.0f;
    ConvRun<IO, W, VEC> run;
    run.load(a, a.x, r, base, t0, lane == 0, true);
    float xe[H + V];  // the H inputs before this run, then the run
    run.values(a.x, base, t0, L, xe + H);
#pragma unroll
    for (int j = 0; j < H; ++j) {
      xe[j] = wave_dpp<kWaveShr1>(xe[V + j]);
      if (lane == 0) xe[j] = run.halo(t0, j);
    }
    float o[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float pre = b;
#pragma unroll
      for (int k = 0; k < W; ++k) pre = fmaf(wk[k], xe[i + k], pre);
      o[i] = a.silu ? silu_f(pre) : pre;
    }
    if (t0 < L) conv_store_run<IO, VEC>(a.out, base, t0, L, o);
  }
}

// The W-1 inputs that end the extended sequence (the state a later call or
// the decode step continues from); one thread per row.  Reads everything it
// needs before writing, so state_out may be state_in.
template <typename IO, int W>
__global__ void __launch_bounds__(256) conv1d_state_kernel(const ConvArgs a, float* state_out) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= a.rows || W == 1) return;
  float v[W > 1 ? W - 1 : 1];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) v[j] = conv_x_at<IO, W>(a, r, a.seqlen - (W - 1) + j);
#pragma unroll
  for (int j = 0; j < W - 1; ++j) state_out[r * (W - 1) + j] = v[j];
}

// One token per row: out = act(bias + sum_k w_k [state, x]_k), state shifted
// in place by one input.  One thread per row.
template <typename IO, int W>
__global__ void __launch_bounds__(256) conv1d_update_kernel(const void* x, float* state,
                                                            const float* w, const float* bias,
                                                            void* out, int64_t rows, int64_t dim,
                                                            int silu) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int64_t d = r % dim;
  float xe[W];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) xe[j] = state[r * (W - 1) + j];
  xe[W - 1] = Io<IO>::ld1(x, r);
  float pre = bias ? bias[d] : 0.0f;
#pragma unroll
  for (int k = 0; k < W; ++k) pre = fmaf(w[d * W + k], xe[k], pre);
  Io<IO>::st1(out, r, silu ? silu_f(pre) : pre);
#pragma unroll
  for (int j = 0; j < W - 1; ++j) state[r * (W - 1) + j] = xe[j + 1];
}

// Backward.  g_t = dout_t silu'(pre_t); dx_s = sum_k w_k g_{s+(W-1)-k};
// dw_k = sum g_t x_{t-(W-1)+k}; dbias = sum g_t; dstate_in from the first
// W-1 outputs.  A thread recomputes pre and g for its V steps and the W-1
// after them (taken from the next lane by a DPP shift, the last lane of the
// wave computes them itself).  dw and dbias are reduced over the workgroup
// (one row per workgroup) and added with one atomic per value.
template <typename IO, int W, bool VEC>
__global__ void __launch_bounds__(256) conv1d_bwd_kernel(const ConvArgs a) {
  constexpr int V = Io<IO>::V, H = W - 1;
  __shared__ float sRed[4][W + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t L = a.seqlen;
  for (int64_t r = blockIdx.y; r < a.rows; r += gridDim.y) {
    const int64_t d = r % a.dim, base = r * L;
    float wk[W];
#pragma unroll
    for (int k = 0; k < W; ++k) wk[k] = a.w[d * W + k];
    const float b = a.bias ? a.bias[d] : 0.0f;
    float dwp[W + 1];
#pragma unroll
    for (int k = 0; k <= W; ++k) dwp[k] = 0.0f;
    // the workgroup walks SELSCAN_CONV_BWD_VPW spans of 256 runs of the row
    for (int it = 0; it < SELSCAN_CONV_BWD_VPW; ++it) {
      const int64_t t0 = (((int64_t)blockIdx.x * SELSCAN_CONV_BWD_VPW + it) * 256 + threadIdx.x) * V;
      if (t0 - threadIdx.x * V >= L) break;  // workgroup-uniform
      // inputs t0-H .. t0+V+H-1 and output gradients t0 .. t0+V+H-1; all loads
      // are issued before the first wait (clamped addresses, values fixed up
      // afterwards)
      ConvRun<IO, W, VEC> rx, rg;
      rx.load(a, a.x, r, base, t0, lane == 0, true);
      rg.load(a, a.dout, r, base, t0, false, false);
      float ax[H > 0 ? H : 1], ag[H > 0 ? H : 1];
      if (lane == 63) {
#pragma unroll
        for (int j = 0; j < H; ++j) {
          const int64_t t = t0 + V + j;
          const int64_t tc = t < L ? t : L - 1;
          ax[j] = Io<IO>::ld1(a.x, base + tc);
          ag[j] = Io<IO>::ld1(a.dout, base + tc);
        }
      }
      float xe[H + V + H], ge[V + H];
      rx.values(a.x, base, t0, L, xe + H);
      rg.values(a.dout, base, t0, L, ge);
#pragma unroll
      for (int j = 0; j < H; ++j) {
        xe[j] = wave_dpp<kWaveShr1>(xe[V + j]);
        xe[H + V + j] = wave_dpp<kWaveShl1>(xe[H + j]);
        ge[V + j] = wave_dpp<kWaveShl1>(ge[j]);
        if (lane == 0) xe[j] = rx.halo(t0, j);
        if (lane == 63) {
          const bool in = t0 + V + j < L;
          xe[H + V + j] = in ? ax[j] : 0.0f;
          ge[V + j] = in ? ag[j] : 0.0f;
        }
      }
      // g for steps t0 .. t0+V+H-1 (zero past L, where dout is zero)
#pragma unroll
      for (int i = 0; i < V + H; ++i) {
        float pre = b;
#pragma unroll
        for (int k = 0; k < W; ++k) pre = fmaf(wk[k], xe[i + k], pre);
        if (a.silu) {
          const float s = rcp(1.0f + ex2(-pre * kLog2e));
          ge[i] *= s * fmaf(pre, 1.0f - s, 1.0f);
        }
      }
      float dxo[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        // own outputs feed dw, dbias
#pragma unroll
        for (int k = 0; k < W; ++k) dwp[k] = fmaf(ge[i], xe[i + k], dwp[k]);
        dwp[W] += ge[i];
        // input t0+i feeds outputs t0+i+H-k
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < W; ++k) acc = fmaf(wk[k], ge[i + H - k], acc);
        dxo[i] = acc;
      }
      if (t0 < L) conv_store_run<IO, VEC>(a.dx, base, t0, L, dxo);
      // the carried inputs before t = 0 feed outputs 0 .. H-1 (first thread of the row)
      if (t0 == 0 && a.dstate_in) {
#pragma unroll
        for (int j = 0; j < H; ++j) {  // input at time j - H
          float acc = 0.0f;
#pragma unroll
          for (int k = 0; k < W; ++k) {
            const int t = j - k;  // output index j - H + H - k
            if (t >= 0) acc = fmaf(wk[k], ge[t], acc);
          }
          a.dstate_in[r * H + j] = acc;
        }
      }
    }
    // workgroup sums of dw and dbias
#pragma unroll
    for (int k = 0; k <= W; ++k) {
      float v = dwp[k];
      v += wave_dpp<kRowShr1>(v);
      v += dpp0<kRowShr2>(v);
      v += dpp0<kRowShr4>(v);
      v += dpp0<kRowShr8>(v);
      v += dpp<kRowBcast15, 0xa>(0.0f, v);
      v += dpp<kRowBcast31, 0xc>(0.0f, v);
      dwp[k] = v;  // lane 63 holds the wave's sum
    }
    if (lane == 63) {
#pragma unroll
      for (int k = 0; k <= W; ++k) sRed[wave][k] = dwp[k];
    }
    __syncthreads();
    if (threadIdx.x <= W) {
      const float s = sRed[0][threadIdx.x] + sRed[1][threadIdx.x] + sRed[2][threadIdx.x] +
                      sRed[3][threadIdx.x];
      if (threadIdx.x < W)
        unsafeAtomicAdd(&a.dw[d * W + threadIdx.x], s);
      else if (a.dbias)
        unsafeAtomicAdd(&a.dbias[d], s);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- Mamba-2 scan (scalar A per head)
//
// With A = a_h I per head the scan becomes block matrix products ("State-
// space models", section "The parallel scan": the restriction of Mamba-2;
// "Structured State Space Models and Mamba ...", section "State Space Duality
// and Mamba-2": Y = (L o Q K^T) V with a 1-semiseparable decay L).  Per
// sequence b, head h and chunk of T = 64 steps, with cs_t the running sum of
// dt A over the chunk and S the state [headdim x N] entering it:
//
//   M[t][s]  = (C_t . B_s) exp(cs_t - cs_s) dt_s     (s <= t, else 0)
//   Y        = M X + diag(exp(cs)) C S^T + D X       (then * silu(z))
//   S'       = exp(cs_63) S + sum_s exp(cs_63 - cs_s) dt_s x_s B_s^T
//
// C . B^T does not depend on the head, so ssd_prep_kernel computes it once
// per (sequence, group, chunk) on MFMA, together with a token-major copy of C.
// ssd_fwd_kernel walks the chunks of one (sequence, head, half of the head
// channels) in order; the three products per chunk run on
// v_mfma_f32_16x16x32_bf16 / v_mfma_f32_32x32x16_bf16 with fp32 accumulation,
// and the state lives in MFMA accumulators for the whole sequence.  Operands
// that are not bf16 inputs (M, the state, the weighted x) are split into a
// bf16 head and a bf16 remainder, v = hi + lo, and multiplied twice, which
// keeps them to about 16 significant bits: a single bf16 rounding of these
// operands alone costs a few percent of |y| on long sequences.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4v_t __attribute__((ext_vector_type(4)));

constexpr int kSsdT = 64;   // steps per chunk
constexpr int kSsdP = 64;   // head channels (headdim)
constexpr int kSsdPB = 32;  // head channels per workgroup

struct SsdArgs {
  const void* x;        // [batch, H * 64, L] bf16
  const void* dt;       // [batch, H, L] bf16, raw
  const float* A;       // [H]
  const void* Bm;       // [batch, G * N, L] bf16
  const void* Cm;
  const float* Dskip;   // [H] or null
  const void* z;        // [batch, H * 64, L] or null
  const float* dt_bias; // [H] or null
  const float* h0;      // [batch, H, 64, N] or null
  void* y;
  float* final_state;   // [batch, H, 64, N] or null
  uint16_t* Ct;         // workspace: [batch, G, nchunks * 64, N] bf16, C token-major
  float* Gf;            // workspace: [batch, G, nchunks, 3, 64, 16] C.B^T tiles, MFMA fragment order
  int64_t batch, L, H, G, N, nchunks;
  int softplus;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += dpp0<kRowShr1>(v);
  v += dpp0<kRowShr2>(v);
  v += dpp0<kRowShr4>(v);
  v += dpp0<kRowShr8>(v);
  v += dpp<kRowBcast15, 0xa>(0.0f, v);
  v += dpp<kRowBcast31, 0xc>(0.0f, v);
  return v;
}

// 8 bf16 of a row (length L) from step t on (t a multiple of 8), read from a
// clamped address: past the end of the row the values are some of the row's
// own (finite) inputs.  The scan never needs them to be zero: every product
// with a step past L is multiplied by that step's dt, which is set to zero,
// and outputs past L are not stored.  ALIGNED (L a multiple of 8, rows
// 16-byte aligned): one 16-byte load; otherwise eight 2-byte loads.  Nothing
// is selected on the loaded values here, so a prefetch is not waited for
// where it is issued.
template <bool ALIGNED>
__device__ __forceinline__ uint4 load8_bf16(const uint16_t* rowp, int64_t t, int64_t L) {
  if constexpr (ALIGNED) {
    return *reinterpret_cast<const uint4*>(rowp + (t < L ? t : L - 8));
  } else {
    uint32_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = rowp[t + j < L ? t + j : L - 1];
    return make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                      e[6] | (e[7] << 16));
  }
}

// Per (sequence, group, chunk): token-major C and the three non-zero 32x32
// tiles of G^T[s][t] = B_s . C_t (s-block <= t-block), stored as each lane's
// 16 accumulators.
template <int N, bool ALIGNED>
__global__ void __launch_bounds__(256) ssd_prep_kernel(const SsdArgs a) {
  constexpr int T = kSsdT, NP = N + 8;
  __shared__ __align__(16) uint16_t sBt[T * NP];
  __shared__ __align__(16) uint16_t sCt[T * NP];
  const int64_t c = blockIdx.x, g = blockIdx.y, b = blockIdx.z, L = a.L, t0 = c * T;
  const uint16_t* Bsrc = static_cast<const uint16_t*>(a.Bm) + (b * a.G + g) * N * L;
  const uint16_t* Csrc = static_cast<const uint16_t*>(a.Cm) + (b * a.G + g) * N * L;
  for (int item = threadIdx.x; item < 2 * N * (T / 8); item += 256) {
    const int tensor = item / (N * (T / 8)), r = item % (N * (T / 8));
    const int n = r / (T / 8), t8 = (r % (T / 8)) * 8;
    const uint4 v = load8_bf16<ALIGNED>((tensor ? Csrc : Bsrc) + n * L, t0 + t8, L);
    uint16_t e[8];
    __builtin_memcpy(e, &v, 16);
    uint16_t* dst = tensor ? sCt : sBt;
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[(t8 + j) * NP + n] = e[j];
  }
  __syncthreads();
  uint16_t* ct = a.Ct + ((b * a.G + g) * a.nchunks * T + t0) * N;
  for (int item = threadIdx.x; item < T * (N / 8); item += 256) {
    const int t = item / (N / 8), n8 = (item % (N / 8)) * 8;
    *reinterpret_cast<uint4*>(ct + t * N + n8) = *reinterpret_cast<const uint4*>(sCt + t * NP + n8);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave < 3) {
    const int sb = wave == 2 ? 1 : 0, tb = wave == 0 ? 0 : 1;  // tiles (0,0), (0,1), (1,1)
    f32x16_t acc = {};
#pragma unroll
    for (int k0 = 0; k0 < N; k0 += 16) {
      const uint4 av = *reinterpret_cast<const uint4*>(sBt + (sb * 32 + lane % 32) * NP + k0 + (lane / 32) * 8);
      const uint4 bv = *reinterpret_cast<const uint4*>(sCt + (tb * 32 + lane % 32) * NP + k0 + (lane / 32) * 8);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(bv), acc, 0, 0, 0);
    }
    float* dst = a.Gf + ((((b * a.G + g) * a.nchunks + c) * 3 + wave) * 64 + lane) * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(dst + 4 * q) =
          make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
  }
}

typedef float f32x2v_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

// two floats rounded to bf16 (nearest even), packed low then high
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const f32x2v_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v_t));
}

// v = hi + lo for two floats: hi their bf16 rounding, lo the bf16 rounding of
// the remainder (about 16 significant bits together)
__device__ __forceinline__ void split_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pk_bf16(a, b);
  lo = pk_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// 8 (4) bf16 of a row at byte offset voff + soff: one 16-byte (8-byte) load
// when rows are 16-byte aligned, else 2-byte loads
template <bool ALIGNED>
__device__ __forceinline__ uint4 buf_ld8_bf16(Rsrc r, uint32_t voff, uint32_t soff) {
  if constexpr (ALIGNED) {
    return buf_ld128(r, voff, soff);
  } else {
    uint32_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = buf_ld16(r, voff + 2 * j, soff);
    return make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
  }
}
template <bool ALIGNED>
__device__ __forceinline__ uint2 buf_ld4_bf16(Rsrc r, uint32_t voff, uint32_t soff) {
  if constexpr (ALIGNED) {
    return buf_ld64(r, voff, soff);
  } else {
    uint32_t e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = buf_ld16(r, voff + 2 * j, soff);
    return make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
  }
}

// One workgroup per (sequence, head, half of the 64 head channels); four
// waves.  Wave w owns the output rows t in [16w, 16w + 16) (two 16x16 tiles
// of Y, one per 16 channels), the state n-blocks w, w + 4, ... (32 x 32
// tiles of S^T) and 12 of the 48 (tile, accumulator) slots of the three
// non-zero 32 x 32 tiles of M.  Per chunk:
//   1. step sizes and running decay (lane = step);
//   2. x and the weighted x (hi, lo) to LDS, M (hi, lo) to LDS;
//   3. Y = C S^T scaled by exp(cs_t), + M X, then D x and the gate; the
//      state update S^T = exp(cs_63) S^T + B^T (w o X);
//   4. the new state (hi, lo) to LDS.
// The operands of chunk c + 1 are loaded into the other register set while
// chunk c is computed; every load of chunk c is waited for at the top of its
// iteration, before anything else is issued, so no store is pending at a
// wait that should only cover loads.
template <int N, bool GATE, bool ALIGNED>
__global__ void __launch_bounds__(256) ssd_fwd_kernel(const SsdArgs a) {
  constexpr int T = kSsdT, PB = kSsdPB, XP = T + 8, SP = N + 8, MP = T + 8;
  constexpr int NB = N / 32, NBW = (NB + 3) / 4;  // state n-blocks, per wave
  __shared__ __align__(16) uint16_t sX[PB * XP];    // x of the chunk, [p][t]
  __shared__ __align__(16) uint16_t sXw[PB * XP];   // w o x, [p][s], bf16 head
  __shared__ __align__(16) uint16_t sXwl[PB * XP];  // and remainder
  __shared__ __align__(16) uint16_t sM[T * MP];     // M[t][s], bf16 head
  __shared__ __align__(16) uint16_t sMl[T * MP];    // and remainder
  __shared__ __align__(16) uint16_t sS[PB * SP];    // S[p][n] entering the chunk, bf16 head
  __shared__ __align__(16) uint16_t sSl[PB * SP];   // and remainder
  // per step: running decay cs (log2 units), step dt, exp(cs), and the
  // weight exp(cs_63 - cs_s) dt_s of step s in the state update
  __shared__ __align__(16) float sCs[T], sDt[T], sE[T], sW[T];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Workgroups are handed to the eight XCDs round-robin in dispatch order;
  // when they divide evenly, XCD x takes one contiguous run of (sequence,
  // half-head) cells, so the operands a sequence's heads share (B, C, C.B^T)
  // are fetched into as few of the per-XCD L2 caches as possible.
  int64_t cell = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  {
    const int64_t total = (int64_t)gridDim.x * gridDim.y;
    if (total % 8 == 0) cell = (cell % 8) * (total / 8) + cell / 8;
  }
  const int64_t h = (cell % gridDim.x) >> 1, pb = (cell % gridDim.x) & 1, b = cell / gridDim.x;
  const int64_t g = h / (a.H / a.G), L = a.L;
  const float Ah2 = a.A[h] * kLog2e;  // decays are kept in log2 units
  const float Dh = a.Dskip ? a.Dskip[h] : 0.0f;
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  const int64_t row0 = (b * a.H * kSsdP + h * kSsdP + pb * PB) * L;  // this workgroup's first channel row
  // buffers: this workgroup's channel rows of x, z, y; its head's steps; its
  // group's B rows, token-major C and C.B^T tiles
  const Rsrc rX = make_rsrc(static_cast<const uint16_t*>(a.x) + row0, PB * L * 2);
  const Rsrc rZ = make_rsrc(GATE ? static_cast<const uint16_t*>(a.z) + row0 : a.x, PB * L * 2);
  const Rsrc rY = make_rsrc(static_cast<uint16_t*>(a.y) + row0, PB * L * 2);
  const Rsrc rDt = make_rsrc(static_cast<const uint16_t*>(a.dt) + (b * a.H + h) * L, L * 2);
  const Rsrc rB = make_rsrc(static_cast<const uint16_t*>(a.Bm) + (b * a.G + g) * N * L, N * L * 2);
  const Rsrc rC = make_rsrc(a.Ct + (b * a.G + g) * a.nchunks * T * N, a.nchunks * T * N * 2);
  const Rsrc rG = make_rsrc(a.Gf + (b * a.G + g) * a.nchunks * 3 * 64 * 16, a.nchunks * 3 * 64 * 16 * 4);
  const int64_t st0 = ((b * a.H + h) * kSsdP + pb * PB) * N;  // state rows of this workgroup

  // ---- state: S^T tiles in accumulators; lane: p = lane % 32, n = nb*32 + row(i)
  // state n-block nb (32 states) of the 32 channels as four 16 x 16 tiles of
  // S^T, tile (ns, pb): lane holds n = nb*32 + ns*16 + (lane/16)*4 + i,
  // p = pb*16 + lane % 16 (four short MFMA chains instead of one long one)
  f32x4v_t S[NBW][2][2];
#pragma unroll
  for (int q = 0; q < NBW; ++q) {
    const int nb = wave + 4 * q;
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
      for (int pb2 = 0; pb2 < 2; ++pb2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = nb * 32 + ns * 16 + (lane / 16) * 4 + i;
          S[q][ns][pb2][i] = (a.h0 && nb < NB) ? a.h0[st0 + (pb2 * 16 + lane % 16) * N + n] : 0.0f;
        }
  }
  auto write_state_bf16 = [&]() {
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
      const int nb = wave + 4 * q;
      if (nb < NB) {
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
          for (int pb2 = 0; pb2 < 2; ++pb2) {
            const int n = nb * 32 + ns * 16 + (lane / 16) * 4, p = pb2 * 16 + lane % 16;
            const f32x4v_t& v4 = S[q][ns][pb2];
            uint2 v, w;
            split_bf16(v4[0], v4[1], v.x, w.x);
            split_bf16(v4[2], v4[3], v.y, w.y);
            *reinterpret_cast<uint2*>(sS + p * SP + n) = v;
            *reinterpret_cast<uint2*>(sSl + p * SP + n) = w;
          }
      }
    }
  };
  write_state_bf16();

  // ---- per-chunk operands, loaded one chunk ahead into the other set
  const int xp = threadIdx.x / 8, xt8 = (threadIdx.x % 8) * 8;  // staging: channel row, 8 steps
  const int ty = 16 * wave + (lane / 16) * 4;                      // first Y row of this lane
  struct Pre {
    uint4 xv;
    uint2 zv[2];           // z at the lane's Y rows, for its two channels
    uint32_t dtr;
    float4 gf[3];          // this wave's 12 slots of C.B^T
    uint4 ct[N / 32];      // C[t = 16 wave + lane % 16][32 k + (lane/16)*8 + j]
    uint4 bt[NBW][4];      // B^T[n = nb*32 + (f/2)*16 + lane % 16][32 (f%2) + (lane/16)*8 + j]
  };
  // per-lane byte offsets; the chunk's offset is added as a scalar.  Reads
  // past the end of a row return another row's (finite) inputs or zero: every
  // product with a step past L is multiplied by that step's dt, which is set
  // to zero, and outputs past L are not stored.
  const uint32_t oX = (uint32_t)((xp * L + xt8) * 2);
  const uint32_t oZ = (uint32_t)(((lane % 16) * L + ty) * 2), oZ16 = (uint32_t)(16 * L * 2);
  const uint32_t oC = (uint32_t)(((16 * wave + lane % 16) * N + (lane / 16) * 8) * 2);
  const uint32_t oB = (uint32_t)(((wave * 32 + lane % 16) * L + (lane / 16) * 8) * 2), oB4 = (uint32_t)(128 * L * 2),
                 oB16 = (uint32_t)(16 * L * 2);
  // the operands of a chunk are loaded piece by piece, each into the
  // registers the previous chunk's copy has just left
  auto fetch_dt = [&](int64_t c, Pre& p) {
    p.dtr = buf_ld16(rDt, lane * 2, (uint32_t)(c * T * 2));  // steps past L are zeroed where used
  };
  auto fetch_x = [&](int64_t c, Pre& p) { p.xv = buf_ld8_bf16<ALIGNED>(rX, oX, (uint32_t)(c * T * 2)); };
  auto fetch_g = [&](int64_t c, Pre& p) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int k = 12 * wave + 4 * q;  // slot: tile k / 16, accumulators k % 16 ..
      p.gf[q] = __builtin_bit_cast(float4, buf_ld128(rG, lane * 64, (uint32_t)((c * 3 + (k >> 4)) * 4096 + (k & 15) * 4)));
    }
  };
  auto fetch_c = [&](int64_t c, Pre& p) {
#pragma unroll
    for (int k = 0; k < N / 32; ++k) p.ct[k] = buf_ld128(rC, oC + 64 * k, (uint32_t)(c * T * N * 2));
  };
  auto fetch_z = [&](int64_t c, Pre& p) {
    if constexpr (GATE) {
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) p.zv[pt] = buf_ld4_bf16<ALIGNED>(rZ, oZ + pt * oZ16, (uint32_t)(c * T * 2));
    }
  };
  auto fetch_b = [&](int64_t c, Pre& p) {
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
      if (wave + 4 * q < NB) {
#pragma unroll
        for (int f = 0; f < 4; ++f)  // (n half, 32-step half)
          p.bt[q][f] = buf_ld8_bf16<ALIGNED>(rB, oB + q * oB4 + (f >> 1) * oB16 + 64 * (f & 1), (uint32_t)(c * T * 2));
      }
    }
  };
  auto fetch = [&](int64_t c, Pre& p) {
    fetch_dt(c, p); fetch_x(c, p); fetch_g(c, p); fetch_c(c, p); fetch_z(c, p); fetch_b(c, p);
  };

  uint2 ypend[2];  // y of the previous chunk, stored after the next prefetch is issued
  auto store_y = [&](int64_t c) {
    const int64_t t = c * T + ty;
    const uint32_t t2 = (uint32_t)(c * T * 2);
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      if (ALIGNED) {
        if (t < L) buf_st64(ypend[pt], rY, oZ + pt * oZ16, t2);
      } else {
        const uint32_t e[2] = {ypend[pt].x, ypend[pt].y};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (t + j < L) buf_st16(e[j / 2] >> (16 * (j % 2)), rY, oZ + pt * oZ16 + 2 * j, t2);
      }
    }
  };

  Pre cur;
  auto chunk = [&](int64_t c) {
    const int64_t t0 = c * T;
    const bool more = c + 1 < a.nchunks;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the operands of chunk c have arrived
    if (c > 0) store_y(c - 1);
    // ---- 1. step sizes and running decay, lane l <-> step t0 + l
    float dtv = 0.0f;
    if (t0 + lane < L) {
      const float raw = __uint_as_float(cur.dtr << 16) + bias;
      dtv = a.softplus ? softplus_f(raw) : raw;
    }
    if (more) fetch_dt(c + 1, cur);
    const float cs = wave_prefix_sum(dtv * Ah2);
    const float cs_end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), T - 1));
    if (wave == 0) {
      sCs[lane] = cs;
      sDt[lane] = dtv;
      sE[lane] = ex2(cs);
      sW[lane] = ex2(cs_end - cs) * dtv;
    }
    __syncthreads();  // A: step data visible; the previous chunk is done with sX, sXw, sM
    // ---- 2. x, w o x and M to LDS
    {
      *reinterpret_cast<uint4*>(sX + xp * XP + xt8) = cur.xv;
      const float4 w0 = *reinterpret_cast<const float4*>(sW + xt8);
      const float4 w1 = *reinterpret_cast<const float4*>(sW + xt8 + 4);
      const uint32_t e[4] = {cur.xv.x, cur.xv.y, cur.xv.z, cur.xv.w};
      const float wj[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        split_bf16(bf_lo(e[j]) * wj[2 * j], bf_hi(e[j]) * wj[2 * j + 1], hi[j], lo[j]);
      *reinterpret_cast<uint4*>(sXw + xp * XP + xt8) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      *reinterpret_cast<uint4*>(sXwl + xp * XP + xt8) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      if (more) fetch_x(c + 1, cur);
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int k = 12 * wave + 4 * q, tile = k >> 4, r = (k & 15) >> 2;
      const int sb = tile == 2 ? 1 : 0, tb = tile == 0 ? 0 : 1;  // tiles (0,0), (0,1), (1,1)
      const int t = tb * 32 + lane % 32, s = sb * 32 + r * 8 + (lane / 32) * 4;
      const float cst = sCs[t];
      const float4 css = *reinterpret_cast<const float4*>(sCs + s);
      const float4 dts = *reinterpret_cast<const float4*>(sDt + s);
      const float csv[4] = {css.x, css.y, css.z, css.w}, dtj[4] = {dts.x, dts.y, dts.z, dts.w};
      const float gv[4] = {cur.gf[q].x, cur.gf[q].y, cur.gf[q].z, cur.gf[q].w};
      float m[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) m[e] = s + e <= t ? gv[e] * ex2(cst - csv[e]) * dtj[e] : 0.0f;
      uint2 v, vl;
      split_bf16(m[0], m[1], v.x, vl.x);
      split_bf16(m[2], m[3], v.y, vl.y);
      *reinterpret_cast<uint2*>(sM + t * MP + s) = v;
      *reinterpret_cast<uint2*>(sMl + t * MP + s) = vl;
    }
    if (more) fetch_g(c + 1, cur);
    __syncthreads();  // B: sX, sXw, sM ready
    // ---- 3a. Y rows t in [16 wave, 16 wave + 16), channels p = pt*16 + lane % 16
    {
      f32x4v_t yv[2] = {{}, {}};
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
        for (int k = 0; k < N / 32; ++k) {
          const int off = (pt * 16 + lane % 16) * SP + 32 * k + (lane / 16) * 8;
          const uint4 sv = *reinterpret_cast<const uint4*>(sS + off);
          const uint4 sl = *reinterpret_cast<const uint4*>(sSl + off);
          yv[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.ct[k]), as_bf16x8(sv), yv[pt], 0, 0, 0);
          yv[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.ct[k]), as_bf16x8(sl), yv[pt], 0, 0, 0);
        }
      }
      if (more) fetch_c(c + 1, cur);
      const float4 ev = *reinterpret_cast<const float4*>(sE + ty);
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        yv[pt][0] *= ev.x; yv[pt][1] *= ev.y; yv[pt][2] *= ev.z; yv[pt][3] *= ev.w;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          if (k == 0 || wave >= 2) {  // M is zero for s > t
            const int mo = (16 * wave + lane % 16) * MP + 32 * k + (lane / 16) * 8;
            const uint4 mv = *reinterpret_cast<const uint4*>(sM + mo);
            const uint4 ml = *reinterpret_cast<const uint4*>(sMl + mo);
            const uint4 xv = *reinterpret_cast<const uint4*>(sX + (pt * 16 + lane % 16) * XP + 32 * k + (lane / 16) * 8);
            yv[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(mv), as_bf16x8(xv), yv[pt], 0, 0, 0);
            yv[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ml), as_bf16x8(xv), yv[pt], 0, 0, 0);
          }
        }
        // epilogue: channel p, steps ty .. ty + 3
        const uint2 xr = *reinterpret_cast<const uint2*>(sX + (pt * 16 + lane % 16) * XP + ty);
        float v[4] = {fmaf(Dh, bf_lo(xr.x), yv[pt][0]), fmaf(Dh, bf_hi(xr.x), yv[pt][1]),
                      fmaf(Dh, bf_lo(xr.y), yv[pt][2]), fmaf(Dh, bf_hi(xr.y), yv[pt][3])};
        if constexpr (GATE) {
          v[0] *= silu_f(bf_lo(cur.zv[pt].x));
          v[1] *= silu_f(bf_hi(cur.zv[pt].x));
          v[2] *= silu_f(bf_lo(cur.zv[pt].y));
          v[3] *= silu_f(bf_hi(cur.zv[pt].y));
        }
        ypend[pt] = make_uint2(pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3]));
      }
      if (more) fetch_z(c + 1, cur);
    }
    // ---- 3b. state: S^T = exp(cs_63) S^T + B^T (w o X)
    {
      const float decay = ex2(cs_end);
#pragma unroll
      for (int q = 0; q < NBW; ++q)
        if (wave + 4 * q < NB)
#pragma unroll
          for (int ns = 0; ns < 2; ++ns)
#pragma unroll
            for (int pb2 = 0; pb2 < 2; ++pb2) S[q][ns][pb2] *= decay;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
        for (int pb2 = 0; pb2 < 2; ++pb2) {
          // w o X as the B operand: lane holds xw[s = 32 ks2 + (lane/16)*8 + j][p = pb2*16 + lane % 16]
          const int xo = (pb2 * 16 + lane % 16) * XP + 32 * ks2 + (lane / 16) * 8;
          const uint4 xw = *reinterpret_cast<const uint4*>(sXw + xo);
          const uint4 xl = *reinterpret_cast<const uint4*>(sXwl + xo);
#pragma unroll
          for (int q = 0; q < NBW; ++q) {
            if (wave + 4 * q < NB) {
#pragma unroll
              for (int ns = 0; ns < 2; ++ns) {
                f32x4v_t& acc = S[q][ns][pb2];
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.bt[q][2 * ns + ks2]), as_bf16x8(xw), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.bt[q][2 * ns + ks2]), as_bf16x8(xl), acc, 0, 0, 0);
              }
            }
          }
        }
      }
      if (more) fetch_b(c + 1, cur);
    }
    __syncthreads();  // C: every wave is done with sS (old state) and the step data
    write_state_bf16();
  };

  fetch(0, cur);
  __syncthreads();  // the initial state is in sS
  for (int64_t c = 0; c < a.nchunks; ++c) chunk(c);
  store_y(a.nchunks - 1);
  if (a.final_state) {
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
      const int nb = wave + 4 * q;
      if (nb < NB) {
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
          for (int pb2 = 0; pb2 < 2; ++pb2) {
            const int n = nb * 32 + ns * 16 + (lane / 16) * 4, p = pb2 * 16 + lane % 16;
            const f32x4v_t& v4 = S[q][ns][pb2];
            *reinterpret_cast<float4*>(a.final_state + st0 + p * N + n) = make_float4(v4[0], v4[1], v4[2], v4[3]);
          }
      }
    }
  }
}

// ---------------------------------------------------------------- decode step

struct StepArgs {
  float* state;
  const void* u;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  const void* z;
  const float* delta_bias;
  void* y;
  int64_t batch, dim, dstate;
  int softplus;
  int vec;  // dstate % 16 == 0 and A 16-byte aligned: the four-lane kernel
};

// One lane per channel, for state rows that the four-lane kernel below does
// not take (dstate not a multiple of 16, or A not 16-byte aligned): the lane
// walks its channel's row element by element, 16 states at a time.
template <typename IO, int RULE, bool GATE>
__global__ void __launch_bounds__(256) state_update_kernel(const StepArgs a) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= a.batch * a.dim) return;
  const int64_t b = c / a.dim, d = c % a.dim;
  const int64_t N = a.dstate;
  const float uu = Io<IO>::ld1(a.u, c);
  const float raw = Io<IO>::ld1(a.delta, c) + (a.delta_bias ? a.delta_bias[d] : 0.0f);
  const float dl = a.softplus ? softplus_log2(raw) : raw * kLog2e;  // delta / ln 2
  const float w = dl * kLn2 * uu;                                   // delta u
  float* st = a.state + c * N;
  const float* Ar = a.A + d * N;
  const int64_t bc = b * N;
  float acc = 0.0f;
  for (int64_t n0 = 0; n0 < N; n0 += 16) {
    const int cnt = (int)((N - n0) < 16 ? (N - n0) : 16);
    float h[16], An[16], Bv[16], Cv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const bool ok = k < cnt;
      h[k] = ok ? st[n0 + k] : 0.0f;
      An[k] = ok ? Ar[n0 + k] : 0.0f;
      Bv[k] = ok ? Io<IO>::ld1(a.Bm, bc + n0 + k) : 0.0f;
      Cv[k] = ok ? Io<IO>::ld1(a.Cm, bc + n0 + k) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float e, x;
      if constexpr (RULE == kRuleDeltaB) {
        e = ex2(dl * An[k]);
        x = w * Bv[k];
      } else if constexpr (RULE == kRuleZoh) {
        e = ex2(dl * An[k]);
        const float coef = zoh_coef(dl * kLn2 * An[k], dl * kLn2, e, An[k] != 0.0f ? rcp(An[k]) : 0.0f);
        x = coef * Bv[k] * uu;
      } else if constexpr (RULE == kRuleEuler) {
        e = fmaf(dl * kLn2, An[k], 1.0f);
        x = w * Bv[k];
      } else {
        const float hx = 0.5f * kLn2 * dl * An[k];
        const float r = rcp(1.0f - hx);
        e = (1.0f + hx) * r;
        x = w * r * Bv[k];
      }
      h[k] = fmaf(e, h[k], x);
      acc = fmaf(Cv[k], h[k], acc);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (k < cnt) st[n0 + k] = h[k];
  }
  float yv = acc + (a.Dskip ? a.Dskip[d] : 0.0f) * uu;
  if constexpr (GATE) yv *= silu_f(Io<IO>::ld1(a.z, c));
  Io<IO>::st1(a.y, c, yv);
}

// Four lanes per channel (dstate a multiple of 16, A 16-byte aligned): lane q
// of a channel owns states 4q .. 4q + 3 of every 16, so each of a wave's
// 16-byte accesses to the state rows and to A covers 16 whole 64-byte rows;
// the readout's four partial sums are added across the lane quad (DPP).  The
// per-token work (step size, gate) is done by all four lanes.
// OFF32 (every element index of the state and of A below 2^31, checked by
// the launcher): the channel split and the element offsets take 32-bit
// arithmetic, in place of 64-bit divisions, products and adds per lane.
template <typename IO, int RULE, bool GATE, bool OFF32>
__global__ void __launch_bounds__(256) state_update4_kernel(const StepArgs a) {
  using Ix = typename std::conditional<OFF32, uint32_t, int64_t>::type;
  const Ix c = (Ix)(((int64_t)blockIdx.x * 256 + threadIdx.x) >> 2);
  const int q = threadIdx.x & 3;
  if ((int64_t)c >= a.batch * a.dim) return;  // the four lanes of a channel leave together
  const Ix dim = (Ix)a.dim, N = (Ix)a.dstate;
  const Ix b = c / dim, d = c - b * dim;
  const float uu = Io<IO>::ld1(a.u, c);
  const float raw = Io<IO>::ld1(a.delta, c) + (a.delta_bias ? a.delta_bias[d] : 0.0f);
  const float dl = a.softplus ? softplus_log2(raw) : raw * kLog2e;  // delta / ln 2
  const float w = dl * kLn2 * uu;                                   // delta u
  float* st = a.state + c * N + 4 * q;
  const float* Ar = a.A + d * N + 4 * q;
  const Ix bc = b * N + 4 * q;
  float acc = 0.0f;
  for (Ix n0 = 0; n0 < N; n0 += 16) {
    const f32x4 s4 = *reinterpret_cast<const f32x4*>(st + n0);
    const float4 a4 = *reinterpret_cast<const float4*>(Ar + n0);
    float h[4] = {s4.x, s4.y, s4.z, s4.w};
    const float An[4] = {a4.x, a4.y, a4.z, a4.w};
    float Bv[4], Cv[4];
    if constexpr (std::is_same<IO, uint16_t>::value) {
      const uint2 bb = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.Bm) + bc + n0);
      const uint2 cc = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.Cm) + bc + n0);
      Bv[0] = bf_lo(bb.x); Bv[1] = bf_hi(bb.x); Bv[2] = bf_lo(bb.y); Bv[3] = bf_hi(bb.y);
      Cv[0] = bf_lo(cc.x); Cv[1] = bf_hi(cc.x); Cv[2] = bf_lo(cc.y); Cv[3] = bf_hi(cc.y);
    } else {
      const float4 bb = *reinterpret_cast<const float4*>(static_cast<const float*>(a.Bm) + bc + n0);
      const float4 cc = *reinterpret_cast<const float4*>(static_cast<const float*>(a.Cm) + bc + n0);
      Bv[0] = bb.x; Bv[1] = bb.y; Bv[2] = bb.z; Bv[3] = bb.w;
      Cv[0] = cc.x; Cv[1] = cc.y; Cv[2] = cc.z; Cv[3] = cc.w;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float e, x;
      if constexpr (RULE == kRuleDeltaB) {
        e = ex2(dl * An[k]);
        x = w * Bv[k];
      } else if constexpr (RULE == kRuleZoh) {
        e = ex2(dl * An[k]);
        const float coef = zoh_coef(dl * kLn2 * An[k], dl * kLn2, e, An[k] != 0.0f ? rcp(An[k]) : 0.0f);
        x = coef * Bv[k] * uu;
      } else if constexpr (RULE == kRuleEuler) {
        e = fmaf(dl * kLn2, An[k], 1.0f);
        x = w * Bv[k];
      } else {
        const float hx = 0.5f * kLn2 * dl * An[k];
        const float r = rcp(1.0f - hx);
        e = (1.0f + hx) * r;
        x = w * r * Bv[k];
      }
      h[k] = fmaf(e, h[k], x);
      acc = fmaf(Cv[k], h[k], acc);
    }
    const f32x4 v = {h[0], h[1], h[2], h[3]};
    *reinterpret_cast<f32x4*>(st + n0) = v;
  }
  // the quad's four partial readouts: swap neighbours, then pairs
  acc += dpp<0xB1, 0xf>(0.0f, acc);  // quad_perm [1, 0, 3, 2]
  acc += dpp<0x4E, 0xf>(0.0f, acc);  // quad_perm [2, 3, 0, 1]
  if (q == 0) {
    float yv = acc + (a.Dskip ? a.Dskip[d] : 0.0f) * uu;
    if constexpr (GATE) yv *= silu_f(Io<IO>::ld1(a.z, c));
    Io<IO>::st1(a.y, c, yv);
  }
}

// ---------------------------------------------------------------- LTI kernel

template <int RULE>
__global__ void __launch_bounds__(256)
    lti_kernel_kernel(const float* A, const float* Bv, const float* Cv, const float* delta,
                      float* K, int64_t dim, int64_t N, int64_t L, int64_t bs, int64_t cs) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t d = blockIdx.y;
  if (k >= L) return;
  const float dt = delta[d];
  float acc = 0.0f;
  for (int64_t n = 0; n < N; ++n) {
    const float An = A[d * N + n];
    float bbar, pk;  // Bbar / B and Abar^k
    if constexpr (RULE <= kRuleZoh) {
      bbar = RULE == kRuleZoh ? zoh_coef(dt * An, dt, ex2(dt * An * kLog2e), An != 0.0f ? rcp(An) : 0.0f) : dt;
      pk = ex2((float)k * (dt * An * kLog2e));  // exp(k dt A)
    } else {
      float ab;
      if constexpr (RULE == kRuleEuler) {
        ab = fmaf(dt, An, 1.0f);
        bbar = dt;
      } else {
        const float r = rcp(1.0f - 0.5f * dt * An);
        ab = (1.0f + 0.5f * dt * An) * r;
        bbar = dt * r;
      }
      // |Abar|^k with the sign of Abar^k (Euler's Abar can be zero or negative)
      const float mag = k == 0 ? 1.0f : ex2((float)k * lg2(fabsf(ab)));
      pk = (ab < 0.0f && (k & 1)) ? -mag : mag;
    }
    bbar *= Bv[d * bs + n];
    acc = fmaf(Cv[d * cs + n] * pk, bbar, acc);
  }
  K[d * L + k] = acc;
}

// ---------------------------------------------------------------- LTI convolution
//
// y[t] = sum_{k<=t} K[k] u[t-k] + D u[t] per (sequence, channel): the
// time-invariant path, where the recurrence collapses into one causal
// convolution with the kernel K_k = C Abar^k Bbar ("State-space models",
// section "Recurrence and convolution").  Direct sum: a workgroup owns 256
// consecutive outputs of one row and walks the inputs before them in
// 256-step tiles, with the tile of u and the 511 kernel lags it needs staged
// in LDS; each thread accumulates its output in float32.
template <typename IO>
__global__ void __launch_bounds__(256) lti_conv_kernel(const float* K, const void* u,
                                                       const float* Dskip, void* y, int64_t dim,
                                                       int64_t L) {
  __shared__ float sU[256];
  __shared__ float sK[512];
  const int64_t t0 = (int64_t)blockIdx.x * 256, d = blockIdx.y, b = blockIdx.z;
  const int64_t row = (b * dim + d) * L;
  const int64_t t = t0 + threadIdx.x;
  const float* Kd = K + d * L;
  float acc = 0.0f;
  // input tiles s0 = t0 - 256 j, j = 0 .. t0 / 256
  for (int64_t s0 = t0; s0 >= 0; s0 -= 256) {
    __syncthreads();  // the previous tile is no longer read
    const int64_t s = s0 + threadIdx.x;
    sU[threadIdx.x] = s < L ? Io<IO>::ld1(u, row + s) : 0.0f;
    // lags k = t - s for t in [t0, t0 + 256), s in [s0, s0 + 256): k in
    // [t0 - s0 - 255, t0 - s0 + 255]; sK[i] = K[t0 - s0 - 255 + i]
    for (int i = threadIdx.x; i < 511; i += 256) {
      const int64_t k = t0 - s0 - 255 + i;
      sK[i] = (k >= 0 && k < L) ? Kd[k] : 0.0f;
    }
    __syncthreads();
    // t - s = (t0 - s0) + threadIdx.x - j  ->  sK index threadIdx.x - j + 255
    if (s0 == t0) {  // the diagonal tile: only s <= t
      for (int j = 0; j <= (int)threadIdx.x; ++j) acc = fmaf(sK[threadIdx.x - j + 255], sU[j], acc);
    } else {
#pragma unroll 8
      for (int j = 0; j < 256; ++j) acc = fmaf(sK[threadIdx.x - j + 255], sU[j], acc);
    }
  }
  if (t < L) {
    const float ut = Io<IO>::ld1(u, row + t);
    Io<IO>::st1(y, row + t, fmaf(Dskip ? Dskip[d] : 0.0f, ut, acc));
  }
}

// ---------------------------------------------------------------- LTI convolution by FFT
//
// The same y = K * u + D u through the frequency domain ("State-space
// models", section "Recurrence and convolution": the kernel computed once and
// applied with an FFT in O(L log L)).  One workgroup per channel: K is
// zero-padded to M >= 2L - 1 points (a power of two, so that the circular
// convolution of length M equals the causal one for t < L) and transformed
// once; the channel's sequences are then taken two at a time as the real and
// imaginary parts of one complex signal (the product with the transform of a
// real kernel is linear, so the inverse returns the two convolutions as the
// real and imaginary parts), transformed, multiplied and transformed back.
//
// Each transform is Stockham's self-sorting formulation: passes of radix 16
// (and one of radix 2, 4 or 8 when log2 M is not a multiple of 4), natural
// order in and out.  A pass over sub-transforms of length Ns reads, for
// butterfly j, the R points j + q M/R, turns them by exp(-2 pi i q k / (Ns R))
// with k = j mod Ns, takes their R-point DFT in registers and writes point q
// to (j - k) R + k + q Ns.  Passes ping-pong between two LDS buffers (one
// barrier each), padded by one point per 16 so that the strided writes of the
// first passes spread over the banks.  The first pass of a forward transform
// reads HBM directly, the last pass of the kernel's transform keeps its
// points in registers (every later transform's last pass produces the same
// points in the same lanes), and the inverse (the forward transform of the
// conjugate, conjugated) writes y from its last pass.
constexpr int kFftMinLog2 = 8, kFftMaxLog2 = 13;  // M from 256 to 8192 points

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}

// cos(pi m / 8) and sin(pi m / 8), m = 0 .. 7
__device__ __forceinline__ constexpr float cos_pi8(int m) {
  return m == 0 ? 1.0f : m == 1 ? 0.92387953f : m == 2 ? 0.70710678f : m == 3 ? 0.38268343f
       : m == 4 ? 0.0f : m == 5 ? -0.38268343f : m == 6 ? -0.70710678f : -0.92387953f;
}
__device__ __forceinline__ constexpr float sin_pi8(int m) {
  return m == 0 ? 0.0f : m == 1 ? 0.38268343f : m == 2 ? 0.70710678f : m == 3 ? 0.92387953f
       : m == 4 ? 1.0f : m == 5 ? 0.92387953f : m == 6 ? 0.70710678f : 0.38268343f;
}

// R-point DFT (R = 2, 4, 8, 16) of values in registers, natural order in and
// out: radix-2 decimation in time over the bit-reversed input; the twiddle of
// a butterfly of span 2s at offset j is exp(-i pi j / s) = exp(-i pi m / 8)
// with m = 8 j / s, a compile-time constant (m = 0 and m = 4, i.e. 1 and -i,
// need no multiply).
template <int R>
__device__ __forceinline__ void dft_reg(float2 (&v)[R]) {
  constexpr int LG = R == 2 ? 1 : R == 4 ? 2 : R == 8 ? 3 : 4;
  static_assert((1 << LG) == R, "radix 2, 4, 8 or 16");
  float2 a[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    int r = 0;
#pragma unroll
    for (int bit = 0; bit < LG; ++bit) r |= ((i >> bit) & 1) << (LG - 1 - bit);
    a[r] = v[i];
  }
#pragma unroll
  for (int s = 1; s < R; s <<= 1) {
#pragma unroll
    for (int k = 0; k < R; k += 2 * s) {
#pragma unroll
      for (int j = 0; j < s; ++j) {
        const int m = j * (8 / s);
        const float2 b = a[k + j + s];
        float2 t;
        if (m == 0) {
          t = b;
        } else if (m == 4) {
          t = make_float2(b.y, -b.x);
        } else {
          const float c = cos_pi8(m), sn = sin_pi8(m);  // (c - i sn) b
          t = make_float2(fmaf(c, b.x, sn * b.y), fmaf(c, b.y, -sn * b.x));
        }
        const float2 x = a[k + j];
        a[k + j] = make_float2(x.x + t.x, x.y + t.y);
        a[k + j + s] = make_float2(x.x - t.x, x.y - t.y);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i) v[i] = a[i];
}

// One Stockham pass of radix R over M points: ld(i) gives point i of the
// input, st(i, value, it, q) takes point i of the output, where it and q name
// the register slot (the thread's it-th butterfly, its q-th point).
template <int R, int M, typename Ld, typename St>
__device__ __forceinline__ void fft_pass(int Ns, Ld ld, St st) {
  constexpr int NBF = M / R, IT = (NBF + 255) / 256;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int j = (int)threadIdx.x + 256 * it;
    if (NBF % 256 == 0 || j < NBF) {
      const int k = j & (Ns - 1);
      float2 v[R];
#pragma unroll
      for (int q = 0; q < R; ++q) v[q] = ld(j + q * NBF);
      if (Ns > 1) {
        float sn, cs;
        sincospif(-2.0f * (float)k / (float)(Ns * R), &sn, &cs);
        const float2 w = make_float2(cs, sn);
        float2 wq = w;
#pragma unroll
        for (int q = 1; q < R; ++q) {
          v[q] = cmul(v[q], wq);
          if (q + 1 < R) wq = cmul(wq, w);
        }
      }
      dft_reg<R>(v);
      const int base = (j - k) * R + k;
#pragma unroll
      for (int q = 0; q < R; ++q) st(base + q * Ns, v[q], it, q);
    }
  }
}

// LDS (2 x 1.0625 M points of 8 bytes) lets two workgroups share a CU up to
// M = 4096; the register budget is held to match
template <typename IO, int LOG2M>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(LOG2M <= 12 ? 2 : 1)))
lti_conv_fft_kernel(const float* K, const void* u,
                                                           const float* Dskip, void* y,
                                                           int64_t batch, int64_t dim, int64_t L) {
  constexpr int M = 1 << LOG2M, P16 = LOG2M / 4, REM = LOG2M % 4;
  constexpr int NP = P16 + (REM ? 1 : 0);   // passes: radix 16, then radix RL
  constexpr int RL = REM ? (1 << REM) : 16;  // radix of the last pass
  constexpr int MP = M + M / 16;             // one pad point per 16
  constexpr int ITL = (M / RL + 255) / 256;  // butterflies per thread in the last pass
  static_assert(NP >= 2, "the first pass is never the last");
  __shared__ float2 sbuf[2][MP];
  const int64_t d = blockIdx.x;
  auto P = [](int i) { return i + (i >> 4); };
  // whole transform: first(i) gives the input, last(i, v, it, q, buf) takes
  // the output (buf: the LDS buffer the last pass does not read); passes
  // write w0 first, then alternate
  auto transform = [&](auto first, auto last, float2* w0, float2* w1) {
    int Ns = 1;
    fft_pass<16, M>(Ns, first, [&](int i, float2 v, int, int) { w0[P(i)] = v; });
    Ns *= 16;
    __syncthreads();
    float2* src = w0;
    float2* dst = w1;
#pragma unroll 1
    for (int p = 1; p < NP - 1; ++p) {
      fft_pass<16, M>(Ns, [&](int i) { return src[P(i)]; },
                      [&](int i, float2 v, int, int) { dst[P(i)] = v; });
      Ns *= 16;
      __syncthreads();
      float2* t = src;
      src = dst;
      dst = t;
    }
    fft_pass<RL, M>(Ns, [&](int i) { return src[P(i)]; },
                    [&](int i, float2 v, int it, int q) { last(i, v, it, q, dst); });
    return dst;
  };

  // HBM rows through buffer resources of extent L: points past L read as
  // zero (the padding) and are not written
  constexpr uint32_t ES = sizeof(IO);
  auto ldv = [](Rsrc r, int i) -> float {
    if constexpr (ES == 2) return __uint_as_float(buf_ld16(r, (uint32_t)i * 2u, 0) << 16);
    else return __uint_as_float(buf_ld32(r, (uint32_t)i * 4u, 0));
  };
  auto stv = [](Rsrc r, int i, float v) {
    if constexpr (ES == 2) buf_st16(__builtin_bit_cast(uint16_t, (__bf16)v), r, (uint32_t)i * 2u, 0);
    else buf_st32(__float_as_uint(v), r, (uint32_t)i * 4u, 0);
  };
  // the kernel's transform, kept where each lane's last pass puts it
  float2 kh[ITL][RL];
  const Rsrc rK = make_rsrc(K + d * L, L * 4);
  transform([&](int i) { return make_float2(__uint_as_float(buf_ld32(rK, (uint32_t)i * 4u, 0)), 0.0f); },
            [&](int, float2 v, int it, int q, float2*) { kh[it][q] = v; }, sbuf[0], sbuf[1]);
  const float Dd = Dskip ? Dskip[d] : 0.0f;
  const float scale = 1.0f / (float)M;
#pragma unroll 1
  for (int64_t b = 0; b < batch; b += 2) {
    const bool two = b + 1 < batch;
    // sequence b + 1 absent: an empty extent reads zeros and drops the writes
    const int64_t row0 = (b * dim + d) * L, row1 = two ? ((b + 1) * dim + d) * L : row0;
    const Rsrc rU0 = make_rsrc(static_cast<const char*>(u) + row0 * ES, L * ES);
    const Rsrc rU1 = make_rsrc(static_cast<const char*>(u) + row1 * ES, two ? L * ES : 0);
    const Rsrc rY0 = make_rsrc(static_cast<char*>(y) + row0 * ES, L * ES);
    const Rsrc rY1 = make_rsrc(static_cast<char*>(y) + row1 * ES, two ? L * ES : 0);
    __syncthreads();  // the previous pair's last pass has read its buffer
    // forward transform of u_b + i u_{b+1}; its last pass multiplies by the
    // kernel's transform and conjugates, into the buffer it does not read
    float2* X = transform(
        [&](int i) { return make_float2(ldv(rU0, i), ldv(rU1, i)); },
        [&](int i, float2 v, int it, int q, float2* buf) {
          const float2 z = cmul(v, kh[it][q]);
          buf[P(i)] = make_float2(z.x, -z.y);
        },
        sbuf[0], sbuf[1]);
    __syncthreads();
    float2* other = X == sbuf[0] ? sbuf[1] : sbuf[0];
    // inverse: conj of the forward transform of the conjugate, over M
    transform([&](int i) { return X[P(i)]; },
              [&](int i, float2 v, int, int, float2*) {
                stv(rY0, i, fmaf(Dd, ldv(rU0, i), v.x * scale));
                stv(rY1, i, fmaf(Dd, ldv(rU1, i), -v.y * scale));
              },
              other, X);
  }
}

// ---------------------------------------------------------------- LTI convolution by FFT, long sequences
//
// Past seqlen 4096 the transforms (M >= 2 seqlen - 1 points) no longer fit in
// LDS, and one workgroup per channel computes them in four steps through a
// workspace in HBM: with M = R x C (R <= 256, C <= 8192) and the padded
// signal x read as an R x C matrix, x[r C + c],
//
//   X[kr + R kc] = sum_c W_C^{c kc} [ W_M^{c kr} sum_r W_R^{r kr} x[r C + c] ]
//
// (column DFTs of length R, a twiddle, row DFTs of length C; W_N =
// exp(-2 pi i / N)).  The spectrum stays in [kr][kc] order: the kernel's and
// the signal's are multiplied element by element in that order, and the
// inverse takes the same steps backwards (row DFTs, the conjugate twiddle,
// column DFTs; each inverse DFT as the conjugate of the forward DFT of the
// conjugate), which returns natural order.  Every pass works on blocks of
// 8192 points in LDS (CB columns of R points, or RB rows of C points) with
// the batched radix-16 Stockham passes below; as in the in-LDS path the
// sequences go two at a time, as the real and imaginary parts of one signal.

// One radix-R Stockham pass over NB transforms of LEN points in LDS buffer s
// (index i at s[i + i / 16]), in place: every thread reads its butterflies'
// points, the block waits, then writes their results.
template <int R, int LEN, int NB, int NTH = 256>
__device__ __forceinline__ void fft_pass_lds(float2* s, int Ns) {
  constexpr int BPT = LEN / R;      // butterflies per transform
  constexpr int NBF = NB * BPT;
  constexpr int IT = (NBF + NTH - 1) / NTH;
  float2 v[IT][R];
  int base[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int j = (int)threadIdx.x + NTH * it;
    if (NBF % NTH == 0 || j < NBF) {
      const int t = j / BPT, jj = j % BPT, k = jj & (Ns - 1);
#pragma unroll
      for (int q = 0; q < R; ++q) {
        const int i = t * LEN + jj + q * BPT;
        v[it][q] = s[i + (i >> 4)];
      }
      if (Ns > 1) {
        float sn, cs;
        sincospif(-2.0f * (float)k / (float)(Ns * R), &sn, &cs);
        const float2 w = make_float2(cs, sn);
        float2 wq = w;
#pragma unroll
        for (int q = 1; q < R; ++q) {
          v[it][q] = cmul(v[it][q], wq);
          if (q + 1 < R) wq = cmul(wq, w);
        }
      }
      dft_reg<R>(v[it]);
      base[it] = t * LEN + (jj - k) * R + k;
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int j = (int)threadIdx.x + NTH * it;
    if (NBF % NTH == 0 || j < NBF) {
#pragma unroll
      for (int q = 0; q < R; ++q) {
        const int i = base[it] + q * Ns;
        s[i + (i >> 4)] = v[it][q];
      }
    }
  }
  __syncthreads();
}

// NB forward DFTs of LEN points each, in place in LDS, natural order in and
// out, by a workgroup of NTH threads
template <int LEN, int NB, int NTH = 256>
__device__ __forceinline__ void fft_lds(float2* s) {
  constexpr int LG = LEN >= 16384 ? 14 : LEN >= 8192 ? 13 : LEN >= 4096 ? 12 : LEN >= 2048 ? 11
                   : LEN >= 1024 ? 10 : LEN >= 512 ? 9 : LEN >= 256 ? 8 : LEN >= 128 ? 7 : 6;
  static_assert((1 << LG) == LEN, "LEN is a power of two, 64 .. 16384");
  constexpr int P16 = LG / 4, REM = LG % 4;
  int Ns = 1;
#pragma unroll 1
  for (int p = 0; p < P16; ++p) {
    fft_pass_lds<16, LEN, NB, NTH>(s, Ns);
    Ns *= 16;
  }
  if constexpr (REM != 0) fft_pass_lds<(1 << REM), LEN, NB, NTH>(s, Ns);
}

constexpr int kFftLongMaxLog2 = 21;  // M up to 2^21 points: seqlen up to 2^20
constexpr int kFftMidLog2 = 14;      // M = 16384 (seqlen 4097 .. 8192): one transform in LDS

// workspace of the long path: per channel the kernel's spectrum and one signal, M complex each
__host__ __device__ constexpr int64_t fft_long_ws_per_channel(int lg) { return (int64_t)2 << lg; }

// LTI convolution for M = 8192 and 16384 points: every transform is one
// in-place FFT of the whole signal in LDS by 1024 threads (four waves per
// SIMD; one workgroup per CU), so the signal makes no trips through HBM
// between passes and no pass waits on a single wave's LDS latency.  The
// kernel's spectrum sits beside the signal in LDS for M = 8192 (2 x 69.6
// KB) and in the workspace for M = 16384 (written once per channel, read
// once per pair of sequences), since neither LDS nor registers hold it there.
// Otherwise as the in-LDS path above: two sequences as the real and imaginary
// parts of one signal, the product with the kernel's spectrum conjugated, and
// the inverse as the conjugate of the forward transform of the conjugate.
template <typename IO, int LOG2M>
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4)))
lti_conv_fft_mid_kernel(const float* K, const void* u, const float* Dskip, void* y, float2* ws,
                        int64_t batch, int64_t dim, int64_t L) {
  static_assert(LOG2M == 13 || LOG2M == kFftMidLog2, "M = 8192 or 16384");
  constexpr int M = 1 << LOG2M, NTH = 1024;
  constexpr bool KS_LDS = LOG2M == 13;
  __shared__ float2 s[M + M / 16];
  __shared__ float2 sk[KS_LDS ? M + M / 16 : 1];
  auto P = [](int i) { return i + (i >> 4); };
  const int64_t d = blockIdx.x;
  float2* Ks = KS_LDS ? nullptr : ws + d * fft_long_ws_per_channel(LOG2M);
  auto ks = [&](int i) -> float2& {
    if constexpr (KS_LDS) return sk[P(i)];
    else return Ks[i];
  };
  constexpr uint32_t ES = sizeof(IO);
  auto ldv = [](Rsrc r, int i) -> float {
    if constexpr (ES == 2) return __uint_as_float(buf_ld16(r, (uint32_t)i * 2u, 0) << 16);
    else return __uint_as_float(buf_ld32(r, (uint32_t)i * 4u, 0));
  };
  auto stv = [](Rsrc r, int i, float v) {
    if constexpr (ES == 2) buf_st16(__builtin_bit_cast(uint16_t, (__bf16)v), r, (uint32_t)i * 2u, 0);
    else buf_st32(__float_as_uint(v), r, (uint32_t)i * 4u, 0);
  };
  // the kernel's spectrum (points past L read as zero through the extent)
  {
    const Rsrc rK = make_rsrc(K + d * L, L * 4);
    for (int i = threadIdx.x; i < M; i += NTH)
      s[P(i)] = make_float2(__uint_as_float(buf_ld32(rK, (uint32_t)i * 4u, 0)), 0.0f);
    __syncthreads();
    fft_lds<M, 1, NTH>(s);
    for (int i = threadIdx.x; i < M; i += NTH) ks(i) = s[P(i)];
  }
  const float Dd = Dskip ? Dskip[d] : 0.0f;
  const float scale = 1.0f / (float)M;
#pragma unroll 1
  for (int64_t b = 0; b < batch; b += 2) {
    const bool two = b + 1 < batch;
    // sequence b + 1 absent: an empty extent reads zeros and drops the writes
    const int64_t row0 = (b * dim + d) * L, row1 = two ? ((b + 1) * dim + d) * L : row0;
    const Rsrc rU0 = make_rsrc(static_cast<const char*>(u) + row0 * ES, L * ES);
    const Rsrc rU1 = make_rsrc(static_cast<const char*>(u) + row1 * ES, two ? L * ES : 0);
    const Rsrc rY0 = make_rsrc(static_cast<char*>(y) + row0 * ES, L * ES);
    const Rsrc rY1 = make_rsrc(static_cast<char*>(y) + row1 * ES, two ? L * ES : 0);
    __syncthreads();  // every thread is done with the buffer's previous contents
    for (int i = threadIdx.x; i < M; i += NTH) s[P(i)] = make_float2(ldv(rU0, i), ldv(rU1, i));
    __syncthreads();
    fft_lds<M, 1, NTH>(s);
    // each thread multiplies the points it then transforms back into place
    for (int i = threadIdx.x; i < M; i += NTH) {
      const float2 z = cmul(s[P(i)], ks(i));
      s[P(i)] = make_float2(z.x, -z.y);
    }
    __syncthreads();
    fft_lds<M, 1, NTH>(s);
    for (int i = threadIdx.x; i < L; i += NTH) {
      const float2 v = s[P(i)];
      stv(rY0, i, fmaf(Dd, ldv(rU0, i), v.x * scale));
      stv(rY1, i, fmaf(Dd, ldv(rU1, i), -v.y * scale));
    }
  }
}


// 512 threads, two workgroups per CU (four waves per SIMD): with 256 threads
// the in-place passes waited on LDS latency.
template <typename IO, int LOG2R, int LOG2C>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4)))
lti_conv_fft_long_kernel(const float* K, const void* u, const float* Dskip, void* y, float2* ws,
                         int64_t batch, int64_t dim, int64_t L) {
  constexpr int R = 1 << LOG2R, C = 1 << LOG2C;
  constexpr int64_t M = (int64_t)R * C;
  constexpr int PB = 8192;                       // points of an LDS block
  constexpr int NTH = 512;                       // threads: one radix-16 butterfly each per pass
  constexpr int CB = PB / R < C ? PB / R : C;    // columns per column block
  constexpr int RB = PB / C < R ? PB / C : R;    // rows per row block
  constexpr int NPT = CB * R;                    // points of a column block
  constexpr int NPR = RB * C;                    // points of a row block
  __shared__ float2 s[PB + PB / 16];
  auto P = [](int i) { return i + (i >> 4); };
  const int64_t d = blockIdx.x;
  float2* Ks = ws + d * fft_long_ws_per_channel(LOG2R + LOG2C);  // [kr][kc] spectrum of K
  float2* Wk = Ks + M;                                            // work matrix
  constexpr uint32_t ES = sizeof(IO);
  auto ldv = [](Rsrc r, int64_t i) -> float {
    if constexpr (ES == 2) return __uint_as_float(buf_ld16(r, (uint32_t)i * 2u, 0) << 16);
    else return __uint_as_float(buf_ld32(r, (uint32_t)i * 4u, 0));
  };
  auto stv = [](Rsrc r, int64_t i, float v) {
    if constexpr (ES == 2) buf_st16(__builtin_bit_cast(uint16_t, (__bf16)v), r, (uint32_t)i * 2u, 0);
    else buf_st32(__float_as_uint(v), r, (uint32_t)i * 4u, 0);
  };
  // twiddle W_M^{e}, e = c kr < M, times v (sign -1: the conjugate)
  auto twiddle = [](float2 v, int64_t e, float sign) {
    float sn, cs;
    sincospif(-2.0f * sign * (float)e / (float)M, &sn, &cs);
    return cmul(v, make_float2(cs, sn));
  };

  // column DFTs + twiddle: x (point n read by get(n), zero at n >= L) -> Wk
  auto column_forward = [&](auto get) {
#pragma unroll 1
    for (int c0 = 0; c0 < C; c0 += CB) {
      for (int i = threadIdx.x; i < NPT; i += NTH) {
        const int r = i / CB, cc = i % CB;  // consecutive threads: consecutive columns
        s[P(cc * R + r)] = get((int64_t)r * C + c0 + cc);
      }
      __syncthreads();
      fft_lds<R, CB, NTH>(s);
      for (int i = threadIdx.x; i < NPT; i += NTH) {
        const int kr = i / CB, cc = i % CB;
        Wk[(int64_t)kr * C + c0 + cc] = twiddle(s[P(cc * R + kr)], (int64_t)(c0 + cc) * kr, 1.0f);
      }
      __syncthreads();
    }
  };

  // the kernel's spectrum: its column pass, then row DFTs stored in Ks
  {
    const Rsrc rK = make_rsrc(K + d * L, L * 4);
    column_forward([&](int64_t n) {
      return make_float2(n < L ? __uint_as_float(buf_ld32(rK, (uint32_t)n * 4u, 0)) : 0.0f, 0.0f);
    });
#pragma unroll 1
    for (int r0 = 0; r0 < R; r0 += RB) {
      for (int i = threadIdx.x; i < NPR; i += NTH) s[P(i)] = Wk[(int64_t)r0 * C + i];
      __syncthreads();
      fft_lds<C, RB, NTH>(s);
      for (int i = threadIdx.x; i < NPR; i += NTH) Ks[(int64_t)r0 * C + i] = s[P(i)];
      __syncthreads();
    }
  }

  const float Dd = Dskip ? Dskip[d] : 0.0f;
  const float scale = 1.0f / (float)M;
#pragma unroll 1
  for (int64_t b = 0; b < batch; b += 2) {
    const bool two = b + 1 < batch;
    const int64_t row0 = (b * dim + d) * L, row1 = two ? ((b + 1) * dim + d) * L : row0;
    const Rsrc rU0 = make_rsrc(static_cast<const char*>(u) + row0 * ES, L * ES);
    const Rsrc rU1 = make_rsrc(static_cast<const char*>(u) + row1 * ES, two ? L * ES : 0);
    const Rsrc rY0 = make_rsrc(static_cast<char*>(y) + row0 * ES, L * ES);
    const Rsrc rY1 = make_rsrc(static_cast<char*>(y) + row1 * ES, two ? L * ES : 0);
    // forward column pass of u_b + i u_{b+1} (points past L: the zero padding,
    // read as zero through the extent L)
    column_forward([&](int64_t n) {
      return n < L ? make_float2(ldv(rU0, n), ldv(rU1, n)) : make_float2(0.0f, 0.0f);
    });
    // row DFTs, product with the kernel's spectrum, inverse row DFTs (as the
    // conjugate of the DFT of the conjugate), conjugate twiddle
#pragma unroll 1
    for (int r0 = 0; r0 < R; r0 += RB) {
      for (int i = threadIdx.x; i < NPR; i += NTH) s[P(i)] = Wk[(int64_t)r0 * C + i];
      __syncthreads();
      fft_lds<C, RB, NTH>(s);
      for (int i = threadIdx.x; i < NPR; i += NTH) {
        const float2 z = cmul(s[P(i)], Ks[(int64_t)r0 * C + i]);
        s[P(i)] = make_float2(z.x, -z.y);
      }
      __syncthreads();
      fft_lds<C, RB, NTH>(s);
      for (int i = threadIdx.x; i < NPR; i += NTH) {
        const int rr = i / C, c = i % C;
        const float2 v = s[P(i)];
        Wk[(int64_t)r0 * C + i] = twiddle(make_float2(v.x, -v.y), (int64_t)c * (r0 + rr), -1.0f);
      }
      __syncthreads();
    }
    // inverse column DFTs; the real and imaginary parts are the two outputs
#pragma unroll 1
    for (int c0 = 0; c0 < C; c0 += CB) {
      for (int i = threadIdx.x; i < NPT; i += NTH) {
        const int kr = i / CB, cc = i % CB;
        const float2 v = Wk[(int64_t)kr * C + c0 + cc];
        s[P(cc * R + kr)] = make_float2(v.x, -v.y);
      }
      __syncthreads();
      fft_lds<R, CB, NTH>(s);
      for (int i = threadIdx.x; i < NPT; i += NTH) {
        const int r = i / CB, cc = i % CB;
        const int64_t n = (int64_t)r * C + c0 + cc;
        if (n < L) {
          const float2 v = s[P(cc * R + r)];  // conj of the result: (v.x, -v.y)
          stv(rY0, n, fmaf(Dd, ldv(rU0, n), v.x * scale));
          stv(rY1, n, fmaf(Dd, ldv(rU1, n), -v.y * scale));
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- host side

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

struct Span {
  const void* p;
  int64_t bytes;
  const char* name;
};

bool overlaps(const Span& x, const Span& y) {
  if (!x.p || !y.p || x.bytes <= 0 || y.bytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)x.p, a1 = a0 + (uintptr_t)x.bytes;
  const uintptr_t b0 = (uintptr_t)y.p, b1 = b0 + (uintptr_t)y.bytes;
  return a0 < b1 && b0 < a1;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int64_t kMaxExtent = (int64_t)1 << 40;
constexpr int64_t kMaxDstate = 64;

int check_extent(const char* name, int64_t v) {
  if (v <= 0 || v > kMaxExtent) return fail(SSM_E_SHAPE, "%s = %lld is out of range", name, (long long)v);
  return SSM_OK;
}

// a * b * c * d <= 2^60 (byte sizes of every tensor stay far from overflow)
bool product_ok(int64_t a, int64_t b, int64_t c = 1, int64_t d = 1) {
  const int64_t lim = (int64_t)1 << 60;
  int64_t p = a;
  for (int64_t f : {b, c, d}) {
    if (p > lim / f) return false;
    p *= f;
  }
  return true;
}

int launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SSM_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return SSM_OK;
}

// calls f with the rule as a compile-time constant
template <typename F>
void with_rule(int rule, F&& f) {
  switch (rule) {
    case kRuleZoh: f(std::integral_constant<int, kRuleZoh>{}); break;
    case kRuleEuler: f(std::integral_constant<int, kRuleEuler>{}); break;
    case kRuleBilinear: f(std::integral_constant<int, kRuleBilinear>{}); break;
    default: f(std::integral_constant<int, kRuleDeltaB>{}); break;
  }
}

template <typename IO, int LPC, int K, int W, int NT, bool VEC>
int launch_fwd_cfg(const ScanArgs& a, int64_t batch, int rule, bool gate, hipStream_t s) {
  constexpr int CPB = (64 / LPC) * W;
  const dim3 grid((unsigned)((a.dim + CPB - 1) / CPB), (unsigned)batch);
  const size_t shmem = 2 * (size_t)CPB * (size_t)a.dstate * sizeof(float);
  // the B/C tiles (static) and the carry and A rows (dynamic, at most
  // kMaxDstate states) must fit one CU's LDS: a layout that cannot fails to
  // compile rather than fault at launch
  constexpr size_t kTiles = 2 * (size_t)NT * LPC * (K + 4) * sizeof(float);
  static_assert(kTiles + 2 * (size_t)CPB * kMaxDstate * sizeof(float) <= kLdsBytes,
                "forward scan layout exceeds the LDS of one CU");
  with_rule(rule, [&](auto rt) {
    constexpr int R = decltype(rt)::value;
    if (gate) hipLaunchKernelGGL((scan_fwd_kernel<IO, LPC, K, W, NT, VEC, R, true>), grid, dim3(64 * W), shmem, s, a);
    else hipLaunchKernelGGL((scan_fwd_kernel<IO, LPC, K, W, NT, VEC, R, false>), grid, dim3(64 * W), shmem, s, a);
  });
  return launch_status("ssm_selective_scan_fwd launch");
}

// The time-pipelined forward for 16 states and bf16 rows (one workgroup per
// 16 channels).
template <bool VEC>
int launch_fwd_pipe(const ScanArgs& a, int64_t batch, int rule, bool gate, hipStream_t s) {
  const dim3 grid((unsigned)((a.dim + 15) / 16), (unsigned)batch);
  auto go = [&](auto rt) {
    constexpr int R = decltype(rt)::value;
    if (gate) hipLaunchKernelGGL((scan_fwd_pipe_kernel<VEC, R, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((scan_fwd_pipe_kernel<VEC, R, false>), grid, dim3(256), 0, s, a);
  };
  if (rule == kRuleEuler) go(std::integral_constant<int, kRuleEuler>{});
  else if (rule == kRuleBilinear) go(std::integral_constant<int, kRuleBilinear>{});
  else go(std::integral_constant<int, kRuleDeltaB>{});
  return launch_status("ssm_selective_scan_fwd launch");
}

// Lane layout choice: 16 lanes per channel gives the shortest cross-lane scan;
// wider groups are used when there are too few channels to give every SIMD of
// the 256 CUs several waves.
template <typename IO, bool VEC>
int launch_fwd_vec(const ScanArgs& a, int64_t batch, int rule, bool gate, hipStream_t s) {
  constexpr int K = SELSCAN_K, W = SELSCAN_W, NT = SELSCAN_NT;
  const int64_t channels = batch * a.dim;
  // The pipelined kernel for bf16 sequences and the rules whose per-element
  // work fits its registers (exact ZOH and float32 rows need more registers
  // than five waves per SIMD leave; the fold-and-scan kernel is faster
  // there).  It addresses a workgroup's 16 rows with 32-bit byte offsets.
  if constexpr (std::is_same<IO, uint16_t>::value) {
    if (rule != kRuleZoh && a.dstate == 16 && channels >= SELSCAN_PIPE_MIN_CHANNELS &&
        16 * a.seqlen * (int64_t)sizeof(IO) < ((int64_t)1 << 31))
      return launch_fwd_pipe<VEC>(a, batch, rule, gate, s);
  }
  if (channels >= 4 * 4096) return launch_fwd_cfg<IO, 16, K, W, NT, VEC>(a, batch, rule, gate, s);
  // 32 lanes per channel: eight waves (16 channels) share each staged
  // 16-state B/C tile
  if (channels >= 2 * 4096) return launch_fwd_cfg<IO, 32, K, 2 * W, NT, VEC>(a, batch, rule, gate, s);
  // 64 lanes per channel: eight waves per workgroup and 8-state tiles, so each
  // staged B/C tile serves 8 channels (at most 2048 waves in such a launch:
  // the grid, not the workgroup size, sets the occupancy)
  return launch_fwd_cfg<IO, 64, K, 2 * W, NT / 2, VEC>(a, batch, rule, gate, s);
}

template <typename IO>
int launch_fwd(const ScanArgs& a, int64_t batch, int rule, bool gate, bool vec, hipStream_t s) {
  return vec ? launch_fwd_vec<IO, true>(a, batch, rule, gate, s)
             : launch_fwd_vec<IO, false>(a, batch, rule, gate, s);
}

// Backward: the gradient pass works on chunks of T = 16 * kBwdK = kCkptT steps.
constexpr int kBwdK = 8;
static_assert(16 * kBwdK == kCkptT, "gradient chunks are the checkpoint blocks");
constexpr int64_t kBwdMaxDstate = kBwdMaxN;

struct BwdLayout {
  int64_t chunks, ckpt_off, carry_off, accB_off, accC_off, psum_off, bytes;
};

BwdLayout bwd_layout(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen) {
  auto up = [](int64_t x) { return (x + 255) & ~(int64_t)255; };
  BwdLayout l;
  const int64_t T = 16 * kBwdK;
  l.chunks = (seqlen + T - 1) / T;
  const int64_t states = batch * dim * l.chunks * dstate * 4;
  const int64_t acc = batch * dstate * seqlen * 4;
  l.ckpt_off = 0;
  l.carry_off = up(states);
  l.accB_off = l.carry_off + up(states);
  l.accC_off = l.accB_off + up(acc);
  l.psum_off = l.accC_off + up(acc);
  // per-step sums carried between the 16-state launches (more than 16 states)
  const int64_t psum = dstate > 16 ? 3 * batch * dim * seqlen * 4 : 0;
  l.bytes = l.psum_off + up(psum);
  return l;
}

template <typename IO, bool VEC, bool ZOH, bool GATE>
int launch_bwd_typed(const ScanArgs& fa, BwdArgs ba, int64_t batch, hipStream_t s) {
  constexpr int K = kBwdK;
  const dim3 grid16((unsigned)((ba.dim + 15) / 16), (unsigned)batch);
  // 1. checkpoints: the state entering every kCkptT-step block (a forward
  // pass), unless the caller brings the forward's; the time-pipelined kernel
  // where the forward would take it
  if (fa.ckpt) {
    bool piped = false;
    if constexpr (std::is_same<IO, uint16_t>::value && !ZOH) {
      if (ba.dstate == 16 && batch * ba.dim >= SELSCAN_PIPE_MIN_CHANNELS &&
          16 * ba.seqlen * (int64_t)sizeof(IO) < ((int64_t)1 << 31)) {
        hipLaunchKernelGGL((scan_fwd_pipe_kernel<VEC, kRuleDeltaB, false, true>),
                           dim3((unsigned)((ba.dim + 15) / 16), (unsigned)batch), dim3(256), 0, s, fa);
        piped = true;
      }
    }
    if (!piped)
      hipLaunchKernelGGL((scan_fwd_kernel<IO, 16, 16, 4, 16, VEC, ZOH ? kRuleZoh : kRuleDeltaB, false, true>), grid16, dim3(256),
                         2 * 16 * (size_t)ba.dstate * sizeof(float), s, fa);
  }
  // 2. adjoint carries at every block end (a reverse pass; time-pipelined
  // where the forward is)
  bool piped = false;
  if constexpr (std::is_same<IO, uint16_t>::value) {
    if (ba.dstate == 16 && batch * ba.dim >= SELSCAN_PIPE_MIN_CHANNELS &&
        16 * ba.seqlen * (int64_t)sizeof(IO) < ((int64_t)1 << 31)) {
      hipLaunchKernelGGL((scan_bwd_carry_pipe_kernel<VEC, GATE>), grid16, dim3(256), 0, s, ba);
      piped = true;
    }
  }
  if (piped) {
  } else if (ba.dstate <= 16) {
    hipLaunchKernelGGL((scan_bwd_carry_kernel<IO, 16, VEC, GATE, false>), grid16, dim3(256), 0, s, ba);
  } else {
    hipLaunchKernelGGL((scan_bwd_carry_kernel<IO, 16, VEC, GATE, true>), grid16, dim3(256), 0, s, ba);
  }
  // 3. gradients, every (sequence, chunk) independently; groups of 4 channels
  const int64_t ngroups = (ba.dim + 3) / 4;
  const int64_t cells = ngroups * ba.chunks * batch;
  int64_t gpb = cells / 4096;  // a few thousand workgroups in total
  if (gpb < 1) gpb = 1;
  if (gpb > ngroups) gpb = ngroups;
  ba.groups_per_block = (int)gpb;
  const dim3 gridm((unsigned)((ngroups + gpb - 1) / gpb), (unsigned)ba.chunks, (unsigned)batch);
  if (ba.dstate <= 16) {
    ba.n0 = 0;
    ba.tile_mode = 0;
    hipLaunchKernelGGL((scan_bwd_main_kernel<IO, K, VEC, ZOH, GATE, false>), gridm, dim3(256), 0, s, ba);
    return SSM_OK;
  }
  // more than 16 states: one launch per 16-state tile, in order on the
  // stream, the per-step sums over states carried from one to the next
  for (int64_t n0 = 0; n0 < ba.dstate; n0 += 16) {
    ba.n0 = (int)n0;
    ba.tile_mode = n0 == 0 ? 1 : (n0 + 16 >= ba.dstate ? 3 : 2);
    hipLaunchKernelGGL((scan_bwd_main_kernel<IO, K, VEC, ZOH, GATE, true>), gridm, dim3(256), 0, s, ba);
  }
  return SSM_OK;
}

template <typename IO>
int launch_bwd(const ScanArgs& fa, const BwdArgs& ba, int64_t batch, bool vec, bool zoh, bool gate,
               hipStream_t s) {
  if (vec) {
    if (zoh) return gate ? launch_bwd_typed<IO, true, true, true>(fa, ba, batch, s)
                         : launch_bwd_typed<IO, true, true, false>(fa, ba, batch, s);
    return gate ? launch_bwd_typed<IO, true, false, true>(fa, ba, batch, s)
                : launch_bwd_typed<IO, true, false, false>(fa, ba, batch, s);
  }
  if (zoh) return gate ? launch_bwd_typed<IO, false, true, true>(fa, ba, batch, s)
                       : launch_bwd_typed<IO, false, true, false>(fa, ba, batch, s);
  return gate ? launch_bwd_typed<IO, false, false, true>(fa, ba, batch, s)
              : launch_bwd_typed<IO, false, false, false>(fa, ba, batch, s);
}

void zero_fill(float* p, int64_t n, hipStream_t s) {
  if (!p || n <= 0) return;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
}


// ---------------------------------------------------------------- causal conv1d: launch

template <typename IO, int W>
void launch_conv_fwd(const ConvArgs& a, bool vec, float* state_out, hipStream_t s) {
  constexpr int V = Io<IO>::V;
  const int64_t nvec = (a.seqlen + V - 1) / V;
  const dim3 grid((unsigned)((nvec + 255) / 256), (unsigned)(a.rows < 65535 ? a.rows : 65535));
  if (vec)
    hipLaunchKernelGGL((conv1d_fwd_kernel<IO, W, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((conv1d_fwd_kernel<IO, W, false>), grid, dim3(256), 0, s, a);
  if (state_out && W > 1)
    hipLaunchKernelGGL((conv1d_state_kernel<IO, W>), dim3((unsigned)((a.rows + 255) / 256)),
                       dim3(256), 0, s, a, state_out);
}

template <typename IO, int W>
void launch_conv_bwd(const ConvArgs& a, bool vec, hipStream_t s) {
  constexpr int V = Io<IO>::V, SPAN = 256 * SELSCAN_CONV_BWD_VPW;
  const int64_t nvec = (a.seqlen + V - 1) / V;
  const dim3 grid((unsigned)((nvec + SPAN - 1) / SPAN), (unsigned)(a.rows < 65535 ? a.rows : 65535));
  if (vec)
    hipLaunchKernelGGL((conv1d_bwd_kernel<IO, W, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((conv1d_bwd_kernel<IO, W, false>), grid, dim3(256), 0, s, a);
}

template <typename F>
void with_width(int64_t width, F&& f) {
  switch (width) {
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 3: f(std::integral_constant<int, 3>{}); break;
    default: f(std::integral_constant<int, 4>{}); break;
  }
}

int conv_common_checks(int64_t batch, int64_t dim, int64_t seqlen, int64_t width, int io_dtype) {
  int st;
  if ((st = check_extent("batch", batch)) || (st = check_extent("dim", dim)) ||
      (st = check_extent("seqlen", seqlen)))
    return st;
  if (width < 1 || width > 4)
    return fail(SSM_E_UNSUPPORTED, "width = %lld: supported widths are 1..4", (long long)width);
  if (!product_ok(batch, dim, seqlen, 4)) return fail(SSM_E_SHAPE, "tensor sizes overflow");
  if (io_dtype != SSM_DTYPE_F32 && io_dtype != SSM_DTYPE_BF16)
    return fail(SSM_E_DTYPE, "io_dtype = %d is not SSM_DTYPE_F32 or SSM_DTYPE_BF16", io_dtype);
  return SSM_OK;
}


// ---------------------------------------------------------------- Mamba-2 scan: launch

struct SsdLayout {
  int64_t nchunks, ct_off, g_off, bytes;
};

SsdLayout ssd_layout(int64_t batch, int64_t seqlen, int64_t ngroups, int64_t dstate) {
  auto up = [](int64_t x) { return (x + 255) & ~(int64_t)255; };
  SsdLayout l;
  l.nchunks = (seqlen + kSsdT - 1) / kSsdT;
  l.ct_off = 0;
  l.g_off = up(batch * ngroups * l.nchunks * kSsdT * dstate * 2);
  l.bytes = l.g_off + up(batch * ngroups * l.nchunks * 3 * 64 * 16 * 4);
  return l;
}

template <int N, bool ALIGNED>
void launch_ssd_aligned(const SsdArgs& a, bool gate, hipStream_t s) {
  hipLaunchKernelGGL((ssd_prep_kernel<N, ALIGNED>),
                     dim3((unsigned)a.nchunks, (unsigned)a.G, (unsigned)a.batch), dim3(256), 0, s, a);
  const dim3 grid((unsigned)(2 * a.H), (unsigned)a.batch);
  if (gate)
    hipLaunchKernelGGL((ssd_fwd_kernel<N, true, ALIGNED>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((ssd_fwd_kernel<N, false, ALIGNED>), grid, dim3(256), 0, s, a);
}

// ALIGNED when every sequence row starts on a 16-byte boundary
template <int N>
void launch_ssd(const SsdArgs& a, bool gate, hipStream_t s) {
  const bool aligned = a.L % 8 == 0 && aligned16(a.x) && aligned16(a.dt) && aligned16(a.Bm) &&
                       aligned16(a.Cm) && aligned16(a.y) && (!a.z || aligned16(a.z));
  if (aligned)
    launch_ssd_aligned<N, true>(a, gate, s);
  else
    launch_ssd_aligned<N, false>(a, gate, s);
}

}  // namespace

// ---------------------------------------------------------------- static scratch
//
// Device memory for ssm_ssd_fwd_noalloc, the Mamba-2 scan for callers that
// cannot allocate: it holds the workspace that ssm_ssd_fwd takes from its
// caller (token-major C and the C.B^T tiles), up to kSsdScratchBytes.  Every
// GPU the library runs on holds its own copy until the process ends; all
// calls on one GPU share it, so such calls must not overlap in time.
constexpr int64_t kSsdScratchBytes = (int64_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kSsdScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The device address of `scratch` on the device that runs `stream` (which
// must be the current device): looked up once per device with
// hipGetSymbolAddress, with that device current.  In host code the array's
// own name is not a device address and is never used.
int scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SSM_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return fail(SSM_E_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if ((int)sdev != dev)
      return fail(SSM_E_HIP, "the stream belongs to device %d, the current device is %d",
                  (int)sdev, dev);
  }
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(SSM_E_HIP, "device %d is beyond the %d this library tracks", dev, kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SSM_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SSM_OK;
}

}  // namespace

// ---------------------------------------------------------------- C ABI

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_last_error(void) { return g_last_error; }

const char* ssm_status_str(int status) {
  switch (status) {
    case SSM_OK: return "ok";
    case SSM_E_NULL: return "required pointer is NULL";
    case SSM_E_SHAPE: return "extent out of range";
    case SSM_E_DTYPE: return "unknown io_dtype or bbar_mode";
    case SSM_E_ALIGN: return "sequence tensor not 16-byte aligned";
    case SSM_E_ALIAS: return "output overlaps an input";
    case SSM_E_UNSUPPORTED: return "unsupported dstate";
    case SSM_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int ssm_selective_scan_fwd(const void* u, const void* delta, const float* A, const void* Bm,
                           const void* Cm, const float* Dskip, const void* z,
                           const float* delta_bias, int delta_softplus, const float* h0, void* y,
                           float* final_state, float* checkpoints, int64_t batch, int64_t dim,
                           int64_t dstate, int64_t seqlen, int io_dtype, int bbar_mode,
                           void* hip_stream) {
  g_last_error[0] = 0;
  if (!u) return fail(SSM_E_NULL, "u is NULL");
  if (!delta) return fail(SSM_E_NULL, "delta is NULL");
  if (!A) return fail(SSM_E_NULL, "A is NULL");
  if (!Bm) return fail(SSM_E_NULL, "B is NULL");
  if (!Cm) return fail(SSM_E_NULL, "C is NULL");
  if (!y) return fail(SSM_E_NULL, "y is NULL");
  int st;
  if ((st = check_extent("batch", batch)) || (st = check_extent("dim", dim)) ||
      (st = check_extent("dstate", dstate)) || (st = check_extent("seqlen", seqlen)))
    return st;
  if (batch > 65535) return fail(SSM_E_SHAPE, "batch = %lld exceeds 65535", (long long)batch);
  if (dim > ((int64_t)1 << 30)) return fail(SSM_E_SHAPE, "dim = %lld exceeds 2^30", (long long)dim);
  if (!product_ok(batch, dim, seqlen, 4) || !product_ok(batch, dim, dstate, 4))
    return fail(SSM_E_SHAPE, "tensor sizes overflow");
  if (io_dtype != SSM_DTYPE_F32 && io_dtype != SSM_DTYPE_BF16)
    return fail(SSM_E_DTYPE, "io_dtype = %d is not SSM_DTYPE_F32 or SSM_DTYPE_BF16", io_dtype);
  if (bbar_mode < SSM_BBAR_DELTA_B || bbar_mode > SSM_DISC_BILINEAR)
    return fail(SSM_E_DTYPE, "bbar_mode = %d is not a known rule", bbar_mode);
  if (dstate > kMaxDstate)
    return fail(SSM_E_UNSUPPORTED, "dstate = %lld is outside 1..%lld", (long long)dstate,
                (long long)kMaxDstate);
  const int64_t es = io_dtype == SSM_DTYPE_BF16 ? 2 : 4;
  const int64_t seq_bytes = batch * dim * seqlen * es;
  const int64_t bc_bytes = batch * dstate * seqlen * es;
  const int64_t st_bytes = batch * dim * dstate * 4;
  const Span in[] = {{u, seq_bytes, "u"},
                     {delta, seq_bytes, "delta"},
                     {A, dim * dstate * 4, "A"},
                     {Bm, bc_bytes, "B"},
                     {Cm, bc_bytes, "C"},
                     {Dskip, dim * 4, "D"},
                     {z, z ? seq_bytes : 0, "z"},
                     {delta_bias, dim * 4, "delta_bias"},
                     {h0, st_bytes, "h0"}};
  const void* seq_ptrs[] = {u, delta, Bm, Cm, z, y};
  const char* seq_names[] = {"u", "delta", "B", "C", "z", "y"};
  for (int i = 0; i < 6; ++i)
    if (seq_ptrs[i] && !aligned16(seq_ptrs[i]))
      return fail(SSM_E_ALIGN, "%s is not 16-byte aligned", seq_names[i]);
  const Span ys{y, seq_bytes, "y"};
  for (const Span& s : in)
    if (overlaps(ys, s)) return fail(SSM_E_ALIAS, "y overlaps %s", s.name);
  if (final_state) {
    const Span fs{final_state, st_bytes, "final_state"};
    if (overlaps(fs, ys)) return fail(SSM_E_ALIAS, "final_state overlaps y");
    for (const Span& s : in) {
      if (s.p == h0 && final_state == h0) continue;  // exact in-place resume
      if (overlaps(fs, s)) return fail(SSM_E_ALIAS, "final_state overlaps %s", s.name);
    }
  }
  if (checkpoints) {
    if (kCkptT % SELSCAN_K != 0)
      return fail(SSM_E_UNSUPPORTED, "checkpoints need steps per lane dividing %d", kCkptT);
    const Span cs{checkpoints, batch * dim * ((seqlen + kCkptT - 1) / kCkptT) * dstate * 4,
                  "checkpoints"};
    if (overlaps(cs, ys)) return fail(SSM_E_ALIAS, "checkpoints overlap y");
    if (final_state && overlaps(cs, Span{final_state, st_bytes, "final_state"}))
      return fail(SSM_E_ALIAS, "checkpoints overlap final_state");
    for (const Span& s : in)
      if (overlaps(cs, s)) return fail(SSM_E_ALIAS, "checkpoints overlap %s", s.name);
  }
  ScanArgs a;
  a.ckpt = checkpoints;
  a.u = u; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dskip = Dskip; a.z = z;
  a.delta_bias = delta_bias; a.h0 = h0; a.y = y; a.final_state = final_state;
  a.dim = dim; a.dstate = dstate; a.seqlen = seqlen;
  a.softplus = delta_softplus ? 1 : 0;
  const bool vec = (seqlen % (io_dtype == SSM_DTYPE_BF16 ? 8 : 4)) == 0;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const bool gate = z != nullptr;
  return io_dtype == SSM_DTYPE_BF16 ? launch_fwd<uint16_t>(a, batch, bbar_mode, gate, vec, s)
                                    : launch_fwd<float>(a, batch, bbar_mode, gate, vec, s);
}

int ssm_state_update(float* state, const void* u, const void* delta, const float* A,
                     const void* Bm, const void* Cm, const float* Dskip, const void* z,
                     const float* delta_bias, int delta_softplus, void* y, int64_t batch,
                     int64_t dim, int64_t dstate, int io_dtype, int bbar_mode, void* hip_stream) {
  g_last_error[0] = 0;
  if (!state) return fail(SSM_E_NULL, "state is NULL");
  if (!u) return fail(SSM_E_NULL, "u is NULL");
  if (!delta) return fail(SSM_E_NULL, "delta is NULL");
  if (!A) return fail(SSM_E_NULL, "A is NULL");
  if (!Bm) return fail(SSM_E_NULL, "B is NULL");
  if (!Cm) return fail(SSM_E_NULL, "C is NULL");
  if (!y) return fail(SSM_E_NULL, "y is NULL");
  int st;
  if ((st = check_extent("batch", batch)) || (st = check_extent("dim", dim)) ||
      (st = check_extent("dstate", dstate)))
    return st;
  if (!product_ok(batch, dim, dstate, 4)) return fail(SSM_E_SHAPE, "tensor sizes overflow");
  if (io_dtype != SSM_DTYPE_F32 && io_dtype != SSM_DTYPE_BF16)
    return fail(SSM_E_DTYPE, "io_dtype = %d is not SSM_DTYPE_F32 or SSM_DTYPE_BF16", io_dtype);
  if (bbar_mode < SSM_BBAR_DELTA_B || bbar_mode > SSM_DISC_BILINEAR)
    return fail(SSM_E_DTYPE, "bbar_mode = %d is not a known rule", bbar_mode);
  if (dstate > kMaxDstate)
    return fail(SSM_E_UNSUPPORTED, "dstate = %lld is outside 1..%lld", (long long)dstate,
                (long long)kMaxDstate);
  if (!aligned16(state)) return fail(SSM_E_ALIGN, "state is not 16-byte aligned");
  if (!aligned16(Bm)) return fail(SSM_E_ALIGN, "B is not 16-byte aligned");
  if (!aligned16(Cm)) return fail(SSM_E_ALIGN, "C is not 16-byte aligned");
  const int64_t es = io_dtype == SSM_DTYPE_BF16 ? 2 : 4;
  const int64_t tok = batch * dim * es, bc = batch * dstate * es;
  const Span st_span{state, batch * dim * dstate * 4, "state"}, ys{y, tok, "y"};
  const Span in[] = {{u, tok, "u"},        {delta, tok, "delta"},   {A, dim * dstate * 4, "A"},
                     {Bm, bc, "B"},        {Cm, bc, "C"},           {Dskip, dim * 4, "D"},
                     {z, z ? tok : 0, "z"}, {delta_bias, dim * 4, "delta_bias"}};
  if (overlaps(ys, st_span)) return fail(SSM_E_ALIAS, "y overlaps state");
  for (const Span& s : in) {
    if (overlaps(ys, s)) return fail(SSM_E_ALIAS, "y overlaps %s", s.name);
    if (overlaps(st_span, s)) return fail(SSM_E_ALIAS, "state overlaps %s", s.name);
  }
  StepArgs a;
  a.state = state; a.u = u; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dskip = Dskip;
  a.z = z; a.delta_bias = delta_bias; a.y = y; a.batch = batch; a.dim = dim; a.dstate = dstate;
  a.softplus = delta_softplus ? 1 : 0;
  a.vec = (dstate % 16 == 0 && aligned16(A)) ? 1 : 0;
  // one lane per channel, or four with 16-byte rows (a.vec)
  const int64_t threads = batch * dim * (a.vec ? 4 : 1);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (grid.x == 0 || (threads + 255) / 256 > 0x7fffffff)
    return fail(SSM_E_SHAPE, "batch * dim too large for one launch");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const bool gate = z != nullptr;
  with_rule(bbar_mode, [&](auto rt) {
    constexpr int R = decltype(rt)::value;
    if (a.vec) {
      // 32-bit element offsets: the largest is a state or A element index
      const bool off32 = batch * dim * dstate < ((int64_t)1 << 31) && dim * dstate < ((int64_t)1 << 31);
      auto go = [&](auto io, auto gt, auto o32) {
        hipLaunchKernelGGL((state_update4_kernel<decltype(io), R, decltype(gt)::value, decltype(o32)::value>),
                           grid, dim3(256), 0, s, a);
      };
      auto go_off = [&](auto io, auto gt) {
        if (off32) go(io, gt, std::true_type{});
        else go(io, gt, std::false_type{});
      };
      auto go_gate = [&](auto io) {
        if (gate) go_off(io, std::true_type{});
        else go_off(io, std::false_type{});
      };
      if (io_dtype == SSM_DTYPE_BF16) go_gate(uint16_t{});
      else go_gate(float{});
    } else if (io_dtype == SSM_DTYPE_BF16) {
      if (gate) hipLaunchKernelGGL((state_update_kernel<uint16_t, R, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((state_update_kernel<uint16_t, R, false>), grid, dim3(256), 0, s, a);
    } else {
      if (gate) hipLaunchKernelGGL((state_update_kernel<float, R, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((state_update_kernel<float, R, false>), grid, dim3(256), 0, s, a);
    }
  });
  return launch_status("ssm_state_update launch");
}

int ssm_lti_kernel(const float* A, const float* Bv, const float* Cv, const float* delta, float* K,
                   int64_t dim, int64_t dstate, int64_t L, int64_t b_row_stride,
                   int64_t c_row_stride, int bbar_mode, void* hip_stream) {
  g_last_error[0] = 0;
  if (!A) return fail(SSM_E_NULL, "A is NULL");
  if (!Bv) return fail(SSM_E_NULL, "B is NULL");
  if (!Cv) return fail(SSM_E_NULL, "C is NULL");
  if (!delta) return fail(SSM_E_NULL, "delta is NULL");
  if (!K) return fail(SSM_E_NULL, "K is NULL");
  int st;
  if ((st = check_extent("dim", dim)) || (st = check_extent("dstate", dstate)) ||
      (st = check_extent("L", L)))
    return st;
  if (dim > 65535) return fail(SSM_E_SHAPE, "dim = %lld exceeds 65535", (long long)dim);
  if (!product_ok(dim, L, 4) || !product_ok(dim, dstate, 4) || L > ((int64_t)1 << 36))
    return fail(SSM_E_SHAPE, "tensor sizes overflow");
  if (b_row_stride < 0 || c_row_stride < 0)
    return fail(SSM_E_SHAPE, "row strides must be >= 0");
  if (bbar_mode < SSM_BBAR_DELTA_B || bbar_mode > SSM_DISC_BILINEAR)
    return fail(SSM_E_DTYPE, "bbar_mode = %d is not a known rule", bbar_mode);
  const Span ks{K, dim * L * 4, "K"};
  const Span in[] = {{A, dim * dstate * 4, "A"},
                     {Bv, ((dim - 1) * b_row_stride + dstate) * 4, "B"},
                     {Cv, ((dim - 1) * c_row_stride + dstate) * 4, "C"},
                     {delta, dim * 4, "delta"}};
  for (const Span& s : in)
    if (overlaps(ks, s)) return fail(SSM_E_ALIAS, "K overlaps %s", s.name);
  const dim3 grid((unsigned)((L + 255) / 256), (unsigned)dim);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  with_rule(bbar_mode, [&](auto rt) {
    constexpr int R = decltype(rt)::value;
    hipLaunchKernelGGL(lti_kernel_kernel<R>, grid, dim3(256), 0, s, A, Bv, Cv, delta, K, dim,
                       dstate, L, b_row_stride, c_row_stride);
  });
  return launch_status("ssm_lti_kernel launch");
}

int64_t ssm_selective_scan_bwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate,
                                              int64_t seqlen) {
  if (batch <= 0 || dim <= 0 || dstate <= 0 || seqlen <= 0) return -1;
  if (!product_ok(batch, dim, seqlen, 4) || !product_ok(batch, dim, dstate, seqlen)) return -1;
  return bwd_layout(batch, dim, dstate, seqlen).bytes;
}

int ssm_selective_scan_bwd(const void* u, const void* delta, const float* A, const void* Bm,
                           const void* Cm, const float* Dskip, const void* z,
                           const float* delta_bias, int delta_softplus, const float* h0,
                           const void* dy, const float* dfinal_state, const float* checkpoints,
                           void* du, void* ddelta,
                           float* dA, void* dB, void* dC, float* dD, void* dz,
                           float* ddelta_bias, float* dh0, void* workspace,
                           int64_t workspace_bytes, int64_t batch, int64_t dim, int64_t dstate,
                           int64_t seqlen, int io_dtype, int bbar_mode, void* hip_stream) {
  g_last_error[0] = 0;
  const struct { const void* p; const char* name; } req[] = {
      {u, "u"}, {delta, "delta"}, {A, "A"}, {Bm, "B"}, {Cm, "C"}, {dy, "dy"}, {du, "du"},
      {ddelta, "ddelta"}, {dA, "dA"}, {dB, "dB"}, {dC, "dC"}, {workspace, "workspace"}};
  for (const auto& r : req)
    if (!r.p) return fail(SSM_E_NULL, "%s is NULL", r.name);
  if (z && !dz) return fail(SSM_E_NULL, "dz is NULL while z is given");
  int st;
  if ((st = check_extent("batch", batch)) || (st = check_extent("dim", dim)) ||
      (st = check_extent("dstate", dstate)) || (st = check_extent("seqlen", seqlen)))
    return st;
  if (batch > 65535) return fail(SSM_E_SHAPE, "batch = %lld exceeds 65535", (long long)batch);
  if (dim > ((int64_t)1 << 30)) return fail(SSM_E_SHAPE, "dim = %lld exceeds 2^30", (long long)dim);
  if (!product_ok(batch, dim, seqlen, 4) || !product_ok(batch, dim, dstate, seqlen))
    return fail(SSM_E_SHAPE, "tensor sizes overflow");
  if (io_dtype != SSM_DTYPE_F32 && io_dtype != SSM_DTYPE_BF16)
    return fail(SSM_E_DTYPE, "io_dtype = %d is not SSM_DTYPE_F32 or SSM_DTYPE_BF16", io_dtype);
  if (bbar_mode < SSM_BBAR_DELTA_B || bbar_mode > SSM_DISC_BILINEAR)
    return fail(SSM_E_DTYPE, "bbar_mode = %d is not a known rule", bbar_mode);
  if (bbar_mode != SSM_BBAR_DELTA_B && bbar_mode != SSM_BBAR_ZOH_EXACT)
    return fail(SSM_E_UNSUPPORTED, "the backward takes the exp rules (bbar_mode 0 or 1), got %d",
                bbar_mode);
  if (dstate > kBwdMaxDstate)
    return fail(SSM_E_UNSUPPORTED, "backward supports dstate 1..%lld, got %lld",
                (long long)kBwdMaxDstate, (long long)dstate);
  const BwdLayout lay = bwd_layout(batch, dim, dstate, seqlen);
  if (lay.chunks > 65535) return fail(SSM_E_SHAPE, "seqlen = %lld is too long", (long long)seqlen);
  if (workspace_bytes < lay.bytes)
    return fail(SSM_E_SHAPE, "workspace holds %lld bytes, needs %lld", (long long)workspace_bytes,
                (long long)lay.bytes);
  const int64_t es = io_dtype == SSM_DTYPE_BF16 ? 2 : 4;
  const int64_t seq = batch * dim * seqlen * es, bc = batch * dstate * seqlen * es;
  const int64_t stb = batch * dim * dstate * 4;
  const void* seq_ptrs[] = {u, delta, Bm, Cm, z, dy, du, ddelta, dB, dC, dz, workspace};
  const char* seq_names[] = {"u", "delta", "B", "C", "z", "dy", "du", "ddelta", "dB", "dC", "dz",
                             "workspace"};
  for (int i = 0; i < 12; ++i)
    if (seq_ptrs[i] && !aligned16(seq_ptrs[i]))
      return fail(SSM_E_ALIGN, "%s is not 16-byte aligned", seq_names[i]);
  const Span ins[] = {{u, seq, "u"},           {delta, seq, "delta"},     {A, dim * dstate * 4, "A"},
                      {Bm, bc, "B"},           {Cm, bc, "C"},             {Dskip, dim * 4, "D"},
                      {z, z ? seq : 0, "z"},   {delta_bias, dim * 4, "delta_bias"},
                      {h0, stb, "h0"},         {dy, seq, "dy"},           {dfinal_state, stb, "dfinal_state"},
                      {checkpoints, batch * dim * lay.chunks * dstate * 4, "checkpoints"}};
  const Span outs[] = {{du, seq, "du"},          {ddelta, seq, "ddelta"},  {dA, dim * dstate * 4, "dA"},
                       {dB, bc, "dB"},           {dC, bc, "dC"},           {dD, dim * 4, "dD"},
                       {dz, z ? seq : 0, "dz"},  {ddelta_bias, dim * 4, "ddelta_bias"},
                       {dh0, stb, "dh0"},        {workspace, lay.bytes, "workspace"}};
  for (const Span& o : outs) {
    for (const Span& i : ins)
      if (overlaps(o, i)) return fail(SSM_E_ALIAS, "%s overlaps %s", o.name, i.name);
    for (const Span& o2 : outs)
      if (&o2 != &o && overlaps(o, o2)) return fail(SSM_E_ALIAS, "%s overlaps %s", o.name, o2.name);
  }
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  char* ws = static_cast<char*>(workspace);
  ScanArgs fa;
  memset(&fa, 0, sizeof fa);
  fa.u = u; fa.delta = delta; fa.A = A; fa.Bm = Bm; fa.Cm = Cm; fa.Dskip = Dskip; fa.z = nullptr;
  fa.delta_bias = delta_bias; fa.h0 = h0; fa.y = nullptr; fa.final_state = nullptr;
  fa.dim = dim; fa.dstate = dstate; fa.seqlen = seqlen; fa.softplus = delta_softplus ? 1 : 0;
  // the forward's checkpoints when the caller has them, else recomputed
  fa.ckpt = checkpoints ? nullptr : reinterpret_cast<float*>(ws + lay.ckpt_off);
  BwdArgs ba;
  memset(&ba, 0, sizeof ba);
  ba.u = u; ba.delta = delta; ba.A = A; ba.Bm = Bm; ba.Cm = Cm; ba.Dskip = Dskip; ba.z = z;
  ba.delta_bias = delta_bias; ba.dy = dy; ba.dfinal = dfinal_state; ba.du = du; ba.ddelta = ddelta;
  ba.dA = dA; ba.dD = dD; ba.dz = dz; ba.ddelta_bias = ddelta_bias; ba.dh0 = dh0;
  ba.ckpt = checkpoints ? checkpoints : fa.ckpt;
  ba.carry = reinterpret_cast<float*>(ws + lay.carry_off);
  ba.accB = reinterpret_cast<float*>(ws + lay.accB_off);
  ba.accC = reinterpret_cast<float*>(ws + lay.accC_off);
  ba.psum = dstate > 16 ? reinterpret_cast<float*>(ws + lay.psum_off) : nullptr;
  ba.dim = dim; ba.dstate = dstate; ba.seqlen = seqlen; ba.chunks = lay.chunks;
  ba.softplus = delta_softplus ? 1 : 0;
  const int64_t nacc = batch * dstate * seqlen;
  zero_fill(ba.accB, nacc, s);
  zero_fill(ba.accC, nacc, s);
  zero_fill(dA, dim * dstate, s);
  zero_fill(dD, dim, s);
  zero_fill(ddelta_bias, dim, s);
  const bool vec = (seqlen % (io_dtype == SSM_DTYPE_BF16 ? 8 : 4)) == 0;
  const bool zoh = bbar_mode == SSM_BBAR_ZOH_EXACT, gate = z != nullptr;
  if (io_dtype == SSM_DTYPE_BF16) {
    launch_bwd<uint16_t>(fa, ba, batch, vec, zoh, gate, s);
  } else {
    launch_bwd<float>(fa, ba, batch, vec, zoh, gate, s);
  }
  int64_t blocks = (nacc + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (io_dtype == SSM_DTYPE_BF16) {
    hipLaunchKernelGGL(store_io_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s, ba.accB, dB, nacc);
    hipLaunchKernelGGL(store_io_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s, ba.accC, dC, nacc);
  } else {
    hipLaunchKernelGGL(store_io_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, ba.accB, dB, nacc);
    hipLaunchKernelGGL(store_io_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, ba.accC, dC, nacc);
  }
  return launch_status("ssm_selective_scan_bwd launch");
}

int ssm_causal_conv1d_fwd(const void* x, const float* weight, const float* bias,
                          const float* state_in, void* out, float* state_out, int64_t batch,
                          int64_t dim, int64_t seqlen, int64_t width, int apply_silu,
                          int io_dtype, void* hip_stream) {
  g_last_error[0] = 0;
  if (!x) return fail(SSM_E_NULL, "x is NULL");
  if (!weight) return fail(SSM_E_NULL, "weight is NULL");
  if (!out) return fail(SSM_E_NULL, "out is NULL");
  int st = conv_common_checks(batch, dim, seqlen, width, io_dtype);
  if (st) return st;
  if (!aligned16(x) || !aligned16(out))
    return fail(SSM_E_ALIGN, "x and out must be 16-byte aligned");
  const int64_t es = io_dtype == SSM_DTYPE_BF16 ? 2 : 4;
  const int64_t seq = batch * dim * seqlen * es, stb = batch * dim * (width - 1) * 4;
  const Span ins[] = {{x, seq, "x"}, {weight, dim * width * 4, "weight"}, {bias, dim * 4, "bias"},
                      {state_in, stb, "state_in"}};
  const Span o{out, seq, "out"}, so{state_out, stb, "state_out"};
  for (const Span& i : ins) {
    if (overlaps(o, i)) return fail(SSM_E_ALIAS, "out overlaps %s", i.name);
    // state_out may be state_in itself (the state is read before it is written)
    if (i.p != state_in && overlaps(so, i)) return fail(SSM_E_ALIAS, "state_out overlaps %s", i.name);
  }
  if (overlaps(o, so)) return fail(SSM_E_ALIAS, "state_out overlaps out");
  if (state_out && state_in && state_out != state_in && overlaps(so, Span{state_in, stb, ""}))
    return fail(SSM_E_ALIAS, "state_out partly overlaps state_in");
  ConvArgs a;
  memset(&a, 0, sizeof a);
  a.x = x; a.w = weight; a.bias = bias; a.state_in = state_in; a.out = out;
  a.rows = batch * dim; a.dim = dim; a.seqlen = seqlen; a.silu = apply_silu ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const bool vec = seqlen % (io_dtype == SSM_DTYPE_BF16 ? 8 : 4) == 0;
  with_width(width, [&](auto wt) {
    constexpr int W = decltype(wt)::value;
    if (io_dtype == SSM_DTYPE_BF16)
      launch_conv_fwd<uint16_t, W>(a, vec, state_out, s);
    else
      launch_conv_fwd<float, W>(a, vec, state_out, s);
  });
  return launch_status("ssm_causal_conv1d_fwd launch");
}

int ssm_causal_conv1d_update(const void* x, float* conv_state, const float* weight,
                             const float* bias, void* out, int64_t batch, int64_t dim,
                             int64_t width, int apply_silu, int io_dtype, void* hip_stream) {
  g_last_error[0] = 0;
  if (!x) return fail(SSM_E_NULL, "x is NULL");
  if (!weight) return fail(SSM_E_NULL, "weight is NULL");
  if (!out) return fail(SSM_E_NULL, "out is NULL");
  if (!conv_state && width > 1) return fail(SSM_E_NULL, "conv_state is NULL");
  int st = conv_common_checks(batch, dim, 1, width, io_dtype);
  if (st) return st;
  const int64_t es = io_dtype == SSM_DTYPE_BF16 ? 2 : 4;
  const Span o{out, batch * dim * es, "out"}, cs{conv_state, batch * dim * (width - 1) * 4, "conv_state"};
  const Span ins[] = {{x, batch * dim * es, "x"}, {weight, dim * width * 4, "weight"},
                      {bias, dim * 4, "bias"}};
  for (const Span& i : ins) {
    if (overlaps(o, i)) return fail(SSM_E_ALIAS, "out overlaps %s", i.name);
    if (overlaps(cs, i)) return fail(SSM_E_ALIAS, "conv_state overlaps %s", i.name);
  }
  if (overlaps(o, cs)) return fail(SSM_E_ALIAS, "out overlaps conv_state");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const int64_t rows = batch * dim;
  const dim3 grid((unsigned)((rows + 255) / 256));
  with_width(width, [&](auto wt) {
    constexpr int W = decltype(wt)::value;
    if (io_dtype == SSM_DTYPE_BF16)
      hipLaunchKernelGGL((conv1d_update_kernel<uint16_t, W>), grid, dim3(256), 0, s, x,
                         conv_state, weight, bias, out, rows, dim, apply_silu ? 1 : 0);
    else
      hipLaunchKernelGGL((conv1d_update_kernel<float, W>), grid, dim3(256), 0, s, x, conv_state,
                         weight, bias, out, rows, dim, apply_silu ? 1 : 0);
  });
  return launch_status("ssm_causal_conv1d_update launch");
}

int ssm_causal_conv1d_bwd(const void* x, const float* weight, const float* bias,
                          const float* state_in, const void* dout, void* dx, float* dweight,
                          float* dbias, float* dstate_in, int64_t batch, int64_t dim,
                          int64_t seqlen, int64_t width, int apply_silu, int io_dtype,
                          void* hip_stream) {
  g_last_error[0] = 0;
  if (!x) return fail(SSM_E_NULL, "x is NULL");
  if (!weight) return fail(SSM_E_NULL, "weight is NULL");
  if (!dout) return fail(SSM_E_NULL, "dout is NULL");
  if (!dx) return fail(SSM_E_NULL, "dx is NULL");
  if (!dweight) return fail(SSM_E_NULL, "dweight is NULL");
  int st = conv_common_checks(batch, dim, seqlen, width, io_dtype);
  if (st) return st;
  if (!aligned16(x) || !aligned16(dout) || !aligned16(dx))
    return fail(SSM_E_ALIGN, "x, dout and dx must be 16-byte aligned");
  const int64_t es = io_dtype == SSM_DTYPE_BF16 ? 2 : 4;
  const int64_t seq = batch * dim * seqlen * es, stb = batch * dim * (width - 1) * 4;
  const Span ins[] = {{x, seq, "x"}, {weight, dim * width * 4, "weight"}, {bias, dim * 4, "bias"},
                      {state_in, stb, "state_in"}, {dout, seq, "dout"}};
  const Span outs[] = {{dx, seq, "dx"}, {dweight, dim * width * 4, "dweight"},
                       {dbias, dim * 4, "dbias"}, {dstate_in, stb, "dstate_in"}};
  for (const Span& o : outs) {
    for (const Span& i : ins)
      if (overlaps(o, i)) return fail(SSM_E_ALIAS, "%s overlaps %s", o.name, i.name);
    for (const Span& o2 : outs)
      if (&o2 != &o && overlaps(o, o2)) return fail(SSM_E_ALIAS, "%s overlaps %s", o.name, o2.name);
  }
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  zero_fill(dweight, dim * width, s);
  zero_fill(dbias, dim, s);
  ConvArgs a;
  memset(&a, 0, sizeof a);
  a.x = x; a.w = weight; a.bias = bias; a.state_in = state_in; a.dout = dout; a.dx = dx;
  a.dw = dweight; a.dbias = dbias; a.dstate_in = dstate_in;
  a.rows = batch * dim; a.dim = dim; a.seqlen = seqlen; a.silu = apply_silu ? 1 : 0;
  const bool vec = seqlen % (io_dtype == SSM_DTYPE_BF16 ? 8 : 4) == 0;
  with_width(width, [&](auto wt) {
    constexpr int W = decltype(wt)::value;
    if (io_dtype == SSM_DTYPE_BF16)
      launch_conv_bwd<uint16_t, W>(a, vec, s);
    else
      launch_conv_bwd<float, W>(a, vec, s);
  });
  return launch_status("ssm_causal_conv1d_bwd launch");
}

int64_t ssm_ssd_workspace_size(int64_t batch, int64_t seqlen, int64_t ngroups, int64_t dstate) {
  if (batch <= 0 || seqlen <= 0 || ngroups <= 0 || dstate <= 0) return -1;
  if (!product_ok(batch, ngroups, seqlen + kSsdT, dstate * 2)) return -1;
  return ssd_layout(batch, seqlen, ngroups, dstate).bytes;
}

// The Mamba-2 scan: validation, then the launches.  `scratch_ws`: the
// workspace is the static scratch (workspace is NULL on entry; its address
// is looked up once the arguments are valid; it overlaps no tensor).
static int ssd_fwd_run(const void* x, const void* dt, const float* A, const void* Bm,
                       const void* Cm, const float* Dskip, const void* z, const float* dt_bias,
                       int dt_softplus, const float* h0, void* y, float* final_state,
                       void* workspace, int64_t workspace_bytes, int64_t batch, int64_t seqlen,
                       int64_t nheads, int64_t headdim, int64_t ngroups, int64_t dstate,
                       int io_dtype, void* hip_stream, bool scratch_ws) {
  const struct { const void* p; const char* name; } req[] = {
      {x, "x"}, {dt, "dt"}, {A, "A"}, {Bm, "B"}, {Cm, "C"}, {y, "y"},
      {scratch_ws ? x : workspace, "workspace"}};
  for (const auto& r : req)
    if (!r.p) return fail(SSM_E_NULL, "%s is NULL", r.name);
  int st;
  if ((st = check_extent("batch", batch)) || (st = check_extent("seqlen", seqlen)) ||
      (st = check_extent("nheads", nheads)) || (st = check_extent("headdim", headdim)) ||
      (st = check_extent("ngroups", ngroups)) || (st = check_extent("dstate", dstate)))
    return st;
  if (nheads % ngroups)
    return fail(SSM_E_SHAPE, "nheads = %lld is not a multiple of ngroups = %lld", (long long)nheads,
                (long long)ngroups);
  if (io_dtype != SSM_DTYPE_BF16)
    return fail(io_dtype == SSM_DTYPE_F32 ? SSM_E_UNSUPPORTED : SSM_E_DTYPE,
                "the Mamba-2 scan takes bf16 inputs (io_dtype = %d)", io_dtype);
  if (headdim != kSsdP)
    return fail(SSM_E_UNSUPPORTED, "headdim = %lld: supported headdim is 64", (long long)headdim);
  if (dstate != 32 && dstate != 64 && dstate != 128 && dstate != 256)
    return fail(SSM_E_UNSUPPORTED, "dstate = %lld: supported are 32, 64, 128, 256", (long long)dstate);
  if (batch > 65535 || ngroups > 65535 || nheads > (1 << 30))
    return fail(SSM_E_SHAPE, "batch, ngroups or nheads too large");
  if (!product_ok(batch, nheads * headdim, seqlen, 2) || !product_ok(batch, nheads * headdim, dstate, 4))
    return fail(SSM_E_SHAPE, "tensor sizes overflow");
  const SsdLayout lay = ssd_layout(batch, seqlen, ngroups, dstate);
  // this bound also keeps every buffer the scan kernel addresses (one group's B
  // rows, its C.B^T tiles, 32 channel rows) below 2^31 bytes
  if (lay.nchunks > 65535) return fail(SSM_E_SHAPE, "seqlen = %lld is too long", (long long)seqlen);
  if (workspace_bytes < lay.bytes) {
    if (scratch_ws)
      return fail(SSM_E_SHAPE, "needs %lld bytes of scratch, the static scratch holds %lld",
                  (long long)lay.bytes, (long long)workspace_bytes);
    return fail(SSM_E_SHAPE, "workspace holds %lld bytes, needs %lld", (long long)workspace_bytes,
                (long long)lay.bytes);
  }
  if (!scratch_ws && !aligned16(workspace))
    return fail(SSM_E_ALIGN, "workspace is not 16-byte aligned");
  const int64_t seq = batch * nheads * headdim * seqlen * 2, bc = batch * ngroups * dstate * seqlen * 2;
  const int64_t stb = batch * nheads * headdim * dstate * 4;
  const Span ins[] = {{x, seq, "x"},        {dt, batch * nheads * seqlen * 2, "dt"},
                      {A, nheads * 4, "A"}, {Bm, bc, "B"},
                      {Cm, bc, "C"},        {Dskip, nheads * 4, "D"},
                      {z, z ? seq : 0, "z"}, {dt_bias, nheads * 4, "dt_bias"},
                      {h0, stb, "h0"}};
  const Span outs[] = {{y, seq, "y"}, {final_state, stb, "final_state"},
                       {workspace, lay.bytes, "workspace"}};
  for (const Span& o : outs) {
    for (const Span& i : ins)
      if (overlaps(o, i)) return fail(SSM_E_ALIAS, "%s overlaps %s", o.name, i.name);
    for (const Span& o2 : outs)
      if (&o2 != &o && overlaps(o, o2)) return fail(SSM_E_ALIAS, "%s overlaps %s", o.name, o2.name);
  }
  if (final_state && !aligned16(final_state))
    return fail(SSM_E_ALIGN, "final_state is not 16-byte aligned");
  if (scratch_ws) {
    const int st2 = scratch_address(static_cast<hipStream_t>(hip_stream), &workspace);
    if (st2 != SSM_OK) return st2;
  }
  SsdArgs a;
  memset(&a, 0, sizeof a);
  a.x = x; a.dt = dt; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dskip = Dskip; a.z = z; a.dt_bias = dt_bias;
  a.h0 = h0; a.y = y; a.final_state = final_state;
  char* ws = static_cast<char*>(workspace);
  a.Ct = reinterpret_cast<uint16_t*>(ws + lay.ct_off);
  a.Gf = reinterpret_cast<float*>(ws + lay.g_off);
  a.batch = batch; a.L = seqlen; a.H = nheads; a.G = ngroups; a.N = dstate; a.nchunks = lay.nchunks;
  a.softplus = dt_softplus ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const bool gate = z != nullptr;
  switch (dstate) {
    case 32: launch_ssd<32>(a, gate, s); break;
    case 64: launch_ssd<64>(a, gate, s); break;
    case 128: launch_ssd<128>(a, gate, s); break;
    default: launch_ssd<256>(a, gate, s); break;
  }
  return launch_status("ssm_ssd_fwd launch");
}

int ssm_ssd_fwd(const void* x, const void* dt, const float* A, const void* Bm, const void* Cm,
                const float* Dskip, const void* z, const float* dt_bias, int dt_softplus,
                const float* h0, void* y, float* final_state, void* workspace,
                int64_t workspace_bytes, int64_t batch, int64_t seqlen, int64_t nheads,
                int64_t headdim, int64_t ngroups, int64_t dstate, int io_dtype,
                void* hip_stream) {
  g_last_error[0] = 0;
  return ssd_fwd_run(x, dt, A, Bm, Cm, Dskip, z, dt_bias, dt_softplus, h0, y, final_state,
                     workspace, workspace_bytes, batch, seqlen, nheads, headdim, ngroups, dstate,
                     io_dtype, hip_stream, false);
}

int64_t ssm_ssd_scratch_bytes(void) { return kSsdScratchBytes; }

int ssm_ssd_fwd_noalloc(const void* x, const void* dt, const float* A, const void* Bm,
                        const void* Cm, const float* Dskip, const void* z, const float* dt_bias,
                        int dt_softplus, const float* h0, void* y, float* final_state,
                        int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t ngroups, int64_t dstate, int io_dtype, void* hip_stream) {
  g_last_error[0] = 0;
  // a size the scratch cannot hold is refused before any HIP call
  if (batch > 0 && seqlen > 0 && ngroups > 0 && dstate > 0 && dstate <= 256 &&
      product_ok(batch, ngroups, seqlen + kSsdT, dstate * 2)) {
    const int64_t need = ssd_layout(batch, seqlen, ngroups, dstate).bytes;
    if (need > kSsdScratchBytes)
      return fail(SSM_E_SHAPE, "needs %lld bytes of scratch, the static scratch holds %lld",
                  (long long)need, (long long)kSsdScratchBytes);
  }
  return ssd_fwd_run(x, dt, A, Bm, Cm, Dskip, z, dt_bias, dt_softplus, h0, y, final_state,
                     nullptr, kSsdScratchBytes, batch, seqlen, nheads, headdim, ngroups, dstate,
                     io_dtype, hip_stream, true);
}

int ssm_lti_conv(const float* K, const void* u, const float* Dskip, void* y, int64_t batch,
                 int64_t dim, int64_t seqlen, int io_dtype, void* hip_stream) {
  g_last_error[0] = 0;
  if (!K) return fail(SSM_E_NULL, "K is NULL");
  if (!u) return fail(SSM_E_NULL, "u is NULL");
  if (!y) return fail(SSM_E_NULL, "y is NULL");
  int st;
  if ((st = check_extent("batch", batch)) || (st = check_extent("dim", dim)) ||
      (st = check_extent("seqlen", seqlen)))
    return st;
  if (batch > 65535 || dim > 65535) return fail(SSM_E_SHAPE, "batch and dim must be <= 65535");
  if (seqlen > ((int64_t)1 << 24)) return fail(SSM_E_SHAPE, "seqlen = %lld is too long", (long long)seqlen);
  if (!product_ok(batch, dim, seqlen, 4)) return fail(SSM_E_SHAPE, "tensor sizes overflow");
  if (io_dtype != SSM_DTYPE_F32 && io_dtype != SSM_DTYPE_BF16)
    return fail(SSM_E_DTYPE, "io_dtype = %d is not SSM_DTYPE_F32 or SSM_DTYPE_BF16", io_dtype);
  const int64_t es = io_dtype == SSM_DTYPE_BF16 ? 2 : 4;
  const Span ys{y, batch * dim * seqlen * es, "y"};
  const Span in[] = {{K, dim * seqlen * 4, "K"}, {u, batch * dim * seqlen * es, "u"},
                     {Dskip, dim * 4, "D"}};
  for (const Span& s : in)
    if (overlaps(ys, s)) return fail(SSM_E_ALIAS, "y overlaps %s", s.name);
  const dim3 grid((unsigned)((seqlen + 255) / 256), (unsigned)dim, (unsigned)batch);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (io_dtype == SSM_DTYPE_BF16)
    hipLaunchKernelGGL(lti_conv_kernel<uint16_t>, grid, dim3(256), 0, s, K, u, Dskip, y, dim, seqlen);
  else
    hipLaunchKernelGGL(lti_conv_kernel<float>, grid, dim3(256), 0, s, K, u, Dskip, y, dim, seqlen);
  return launch_status("ssm_lti_conv launch");
}

int64_t ssm_lti_conv_fft_workspace_size(int64_t dim, int64_t seqlen) {
  if (dim <= 0 || seqlen <= 0 || dim > ((int64_t)1 << 30)) return -1;
  int lg = kFftMinLog2;
  while ((int64_t(1) << lg) < 2 * seqlen - 1) ++lg;
  if (lg <= kFftMaxLog2) return 0;
  if (lg > kFftLongMaxLog2) return -1;
  return dim * fft_long_ws_per_channel(lg) * (int64_t)sizeof(float2);
}

int ssm_lti_conv_fft(const float* K, const void* u, const float* Dskip, void* y, void* workspace,
                     int64_t workspace_bytes, int64_t batch, int64_t dim, int64_t seqlen,
                     int io_dtype, void* hip_stream) {
  g_last_error[0] = 0;
  if (!K) return fail(SSM_E_NULL, "K is NULL");
  if (!u) return fail(SSM_E_NULL, "u is NULL");
  if (!y) return fail(SSM_E_NULL, "y is NULL");
  int st;
  if ((st = check_extent("batch", batch)) || (st = check_extent("dim", dim)) ||
      (st = check_extent("seqlen", seqlen)))
    return st;
  if (dim > ((int64_t)1 << 30)) return fail(SSM_E_SHAPE, "dim = %lld exceeds 2^30", (long long)dim);
  if (!product_ok(batch, dim, seqlen, 4)) return fail(SSM_E_SHAPE, "tensor sizes overflow");
  if (io_dtype != SSM_DTYPE_F32 && io_dtype != SSM_DTYPE_BF16)
    return fail(SSM_E_DTYPE, "io_dtype = %d is not SSM_DTYPE_F32 or SSM_DTYPE_BF16", io_dtype);
  int lg = kFftMinLog2;
  while ((int64_t(1) << lg) < 2 * seqlen - 1) ++lg;
  if (lg > kFftLongMaxLog2)
    return fail(SSM_E_UNSUPPORTED, "seqlen = %lld: the FFT path takes seqlen up to %d",
                (long long)seqlen, 1 << (kFftLongMaxLog2 - 1));
  const bool long_path = lg > kFftMaxLog2;
  const int64_t ws_need = long_path ? dim * fft_long_ws_per_channel(lg) * (int64_t)sizeof(float2) : 0;
  if (long_path) {
    if (!workspace)
      return fail(SSM_E_NULL, "workspace is NULL: seqlen = %lld needs %lld bytes of it",
                  (long long)seqlen, (long long)ws_need);
    if (workspace_bytes < ws_need)
      return fail(SSM_E_SHAPE, "workspace holds %lld bytes, needs %lld", (long long)workspace_bytes,
                  (long long)ws_need);
    if (!aligned16(workspace)) return fail(SSM_E_ALIGN, "workspace is not 16-byte aligned");
  }
  const int64_t es = io_dtype == SSM_DTYPE_BF16 ? 2 : 4;
  const Span ys{y, batch * dim * seqlen * es, "y"};
  const Span ws{long_path ? workspace : nullptr, ws_need, "workspace"};
  const Span in[] = {{K, dim * seqlen * 4, "K"}, {u, batch * dim * seqlen * es, "u"},
                     {Dskip, dim * 4, "D"}};
  for (const Span& s : in) {
    if (overlaps(ys, s)) return fail(SSM_E_ALIAS, "y overlaps %s", s.name);
    if (overlaps(ws, s)) return fail(SSM_E_ALIAS, "workspace overlaps %s", s.name);
  }
  if (overlaps(ws, ys)) return fail(SSM_E_ALIAS, "workspace overlaps y");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const bool bf = io_dtype == SSM_DTYPE_BF16;
  auto go = [&](auto lg_tag) {
    constexpr int LG = decltype(lg_tag)::value;
    if (bf)
      hipLaunchKernelGGL((lti_conv_fft_kernel<uint16_t, LG>), dim3((unsigned)dim), dim3(256), 0, s,
                         K, u, Dskip, y, batch, dim, seqlen);
    else
      hipLaunchKernelGGL((lti_conv_fft_kernel<float, LG>), dim3((unsigned)dim), dim3(256), 0, s,
                         K, u, Dskip, y, batch, dim, seqlen);
  };
  // long path: M = R x C with R = 2^min(8, lg / 2), C = M / R <= 8192
  auto go_long = [&](auto lg_tag) {
    constexpr int LG = decltype(lg_tag)::value;
    constexpr int LR = LG / 2 < 8 ? LG / 2 : 8, LC = LG - LR;
    float2* w = static_cast<float2*>(workspace);
    if (bf)
      hipLaunchKernelGGL((lti_conv_fft_long_kernel<uint16_t, LR, LC>), dim3((unsigned)dim), dim3(512),
                         0, s, K, u, Dskip, y, w, batch, dim, seqlen);
    else
      hipLaunchKernelGGL((lti_conv_fft_long_kernel<float, LR, LC>), dim3((unsigned)dim), dim3(512),
                         0, s, K, u, Dskip, y, w, batch, dim, seqlen);
  };
  switch (lg) {
    case 8: go(std::integral_constant<int, 8>{}); break;
    case 9: go(std::integral_constant<int, 9>{}); break;
    case 10: go(std::integral_constant<int, 10>{}); break;
    case 11: go(std::integral_constant<int, 11>{}); break;
    case 12: go(std::integral_constant<int, 12>{}); break;
    case 13:  // one in-LDS transform per signal, the kernel's spectrum beside it
      if (bf)
        hipLaunchKernelGGL((lti_conv_fft_mid_kernel<uint16_t, 13>), dim3((unsigned)dim), dim3(1024), 0, s,
                           K, u, Dskip, y, nullptr, batch, dim, seqlen);
      else
        hipLaunchKernelGGL((lti_conv_fft_mid_kernel<float, 13>), dim3((unsigned)dim), dim3(1024), 0, s,
                           K, u, Dskip, y, nullptr, batch, dim, seqlen);
      break;
    case 14:  // one in-LDS transform per signal (kernel spectrum in the workspace)
      if (bf)
        hipLaunchKernelGGL((lti_conv_fft_mid_kernel<uint16_t, 14>), dim3((unsigned)dim), dim3(1024), 0, s,
                           K, u, Dskip, y, static_cast<float2*>(workspace), batch, dim, seqlen);
      else
        hipLaunchKernelGGL((lti_conv_fft_mid_kernel<float, 14>), dim3((unsigned)dim), dim3(1024), 0, s,
                           K, u, Dskip, y, static_cast<float2*>(workspace), batch, dim, seqlen);
      break;
    case 15: go_long(std::integral_constant<int, 15>{}); break;
    case 16: go_long(std::integral_constant<int, 16>{}); break;
    case 17: go_long(std::integral_constant<int, 17>{}); break;
    case 18: go_long(std::integral_constant<int, 18>{}); break;
    case 19: go_long(std::integral_constant<int, 19>{}); break;
    case 20: go_long(std::integral_constant<int, 20>{}); break;
    default: go_long(std::integral_constant<int, 21>{}); break;
  }
  return launch_status("ssm_lti_conv_fft launch");
}

}  // extern "C"
