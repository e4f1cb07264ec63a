// MoE verify-block library for gfx950 (CDNA4). C ABI in include/moe_verify.h.
//
// One MoE layer over a speculative block of k <= 16 tokens ("Speculating on a Strix Halo",
// sections "Speculative decoding", "What the pieces cost", "The verify's own cost") runs as two
// stream-ordered launches (many sequences at once, up to 1024 tokens: the gathered path further
// down):
//
//   k_router    (expert tile, H slice) items: fp32 MFMA partial logits and sums of squares; the
//               block is also packed as the experts' B operands (bf16 hi/lo fragments, or MX-fp8
//               hi/lo operands for mxfp4 routed experts). Zeroes the counters of k_layer.
//   k_layer     three phases, each starting when the previous one is complete on every workgroup:
//               (1) the routing in LDS (RMSNorm factor, logits, top-K per token with ties to the
//               lower expert, softmax over the K, the woken-expert union by wave ballot + prefix
//               count, the weight table), then (woken expert, row tile) items, assigned statically
//               and balanced, the last rounds claimed: the expert's gate and up rows are streamed
//               from HBM once (128-bit nontemporal loads, the next item prefetched) and applied to
//               all 16 token columns on the matrix cores; SwiGLU, the routing weight and the hi/lo
//               split are fused into the epilogue, which writes the down B operand; (2) (woken
//               expert, row group) items: W_down streamed once, partial rows per (token, slot);
//               (3) the combine y[t] = sum_j P[t, j] + P[t, shared] (+ x[t]), fixed slot order.
//
// The router's results reach k_layer through a kernel boundary. Inside k_layer the phases publish
// through device-coherent stores and counters (no kernel waits on data of a later phase).
//
// Tokens are the MFMA N dimension (16 columns; unused columns are explicit zeros written every
// call), expert rows the M dimension, the hidden / intermediate size the K dimension. MFMA work
// is free next to the HBM stream, so every expert is applied to all 16 columns; columns of tokens
// not routed to it carry weight 0. Activations enter as hi + lo pairs: bf16 (~2^-17 relative)
// against bf16 weights, MX-fp8 (e4m3 with a scale per 32 values) against mxfp4 weights.
//
// K-index mapping of the bf16 MFMA tiles: the reduction dimension is cut into windows of 128; in
// window w, k-step j (0..3), lane l = c + 16 q (c = row or token column, q = 0..3) holds the 8
// values at 128 w + 32 j + 8 q + (0..7) (a lane quad reads 64 contiguous bytes per row and
// instruction). mxfp4 weights go to the scaled instruction whole: in window w lane l holds the
// 32-value block 4 w + q of row c and its scale byte (see the MX-fp8 helpers for the B side).
#include <hip/hip_runtime.h>
#include <algorithm>
#include <atomic>
#include <chrono>
#include <mutex>
#include <random>
#include <type_traits>
#include <stdint.h>
#include <string.h>

#include "moe_verify.h"

namespace {

constexpr int KMAX = 16;          // block tokens = MFMA N
constexpr int WIN = 128;          // reduction window
constexpr int NW = 8;             // waves per workgroup
constexpr int NTH = NW * 64;      // threads per workgroup
constexpr int MAX_E = 512;
constexpr int MAX_K = 16;
constexpr int MAX_U = KMAX * MAX_K;  // woken experts at most
constexpr int HS_MAX = 4;            // H slices of the router at most
static_assert(MAX_E <= NTH, "routing assigns one expert per thread");
constexpr int GU_MX_RT = 2;  // gate/up row tiles per mxfp4 item (bf16: 1); even, <= 4
constexpr int AM_CHUNK = 8192;    // argmax values per workgroup


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Buffer loads for the weight streams: an SGPR resource per tensor, a per-lane constant VGPR
// offset, the tile step as an immediate and the item offset in an SGPR, so the streaming loops do
// no per-load address arithmetic in VGPRs. Loads are nontemporal; offsets past `bytes` read 0.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int BUF_NT = 2;
__device__ __forceinline__ rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, BUF_NT);
}
// cached (the down kernel's activation fragments are re-read by every row group of an expert)
__device__ __forceinline__ u32x4 bld16_cached(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t bld1(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, BUF_NT);
}
__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }

// Device-coherent (sc1) stores and loads: written through to memory and read from it, past the
// XCD-local L2, so data one workgroup publishes inside a launch is visible to workgroups on every
// XCD once the writer's stores are complete (s_waitcnt) and a counter says so; no L2 write-back
// or invalidate fence is needed. A relaxed agent-scope atomic store is exactly such a store.
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
constexpr int BUF_DEV = 16;  // buffer-instruction cache policy bit sc1 (device scope)

__device__ __forceinline__ uint32_t bf16_rne(float f) {  // finite inputs
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// f ~= hi + lo with both halves bf16.
__device__ __forceinline__ void split_bf16(float f, uint32_t& hi, uint32_t& lo) {
  hi = bf16_rne(f);
  lo = bf16_rne(f - __uint_as_float(hi << 16));
}

__device__ __forceinline__ void pack8(const uint32_t (&v)[8], u32x4& o) {
  o.x = v[0] | (v[1] << 16); o.y = v[2] | (v[3] << 16); o.z = v[4] | (v[5] << 16); o.w = v[6] | (v[7] << 16);
}

__device__ __forceinline__ float e8m0_scale(uint32_t byte) { return __uint_as_float(byte << 23); }

// ---- MX-fp8 operands of the scaled matrix-core instruction (mxfp4 layers) ----
// v_mfma_scale_f32_16x16x128_f8f6f4 multiplies a 16x128 A by a 128x16 B with one e8m0 scale per
// 32 values along K for each row of A and each column of B. A (fp4 codes): lane l holds row
// l % 16, K = 32 (l / 16) .. +31, low nibble first, the tiled mxfp4 layout's lane block. B
// (fp8 e4m3): lane l = c + 16 q holds column c at K = 16 q + j in bytes j < 16 and at
// K = 64 + 16 q + j in bytes 16 + j. The scale of (row or column c, 32-block b) is the selected
// byte of lane c + 16 b's scale register. Activations enter as hi + lo fp8 pairs, each with its
// own block scale (the lo part quantises the residual of the hi part).
typedef int v8i __attribute__((ext_vector_type(8)));
constexpr int MXW = 4096 + 256;  // bytes per 128-wide window: hi [64][32], lo [64][32], scales [64] u32

// e8m0 exponent for a block whose largest magnitude is m: the smallest e with m 2^-e <= 448 (the
// largest e4m3 value), clamped to [-127, 127]; an all-zero block takes -127.
__device__ __forceinline__ int mx8_exp(float m) {
  if (!(m > 0.f)) return -127;
  int e = (int)((__float_as_uint(m) >> 23) & 0xFFu) - 127 - 8;
  if (ldexpf(m, -e) > 448.f) ++e;
  return max(-127, min(127, e));
}
// four values to e4m3 (round to nearest even), packed low to high
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
// N values (a multiple of 4) as hi and lo fp8 words with their exponents; the block maximum is
// taken over the values and, when PARTNER is set, over the same computation in lane ^ 16.
template <int N, bool PARTNER>
__device__ __forceinline__ void mx8_quant(const float (&v)[N], uint32_t (&hi)[N / 4], uint32_t (&lo)[N / 4],
                                          int& eh, int& el) {
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < N; ++j) m = fmaxf(m, fabsf(v[j]));
  if (PARTNER) m = fmaxf(m, __shfl_xor(m, 16));
  eh = mx8_exp(m);
#pragma unroll
  for (int g = 0; g < N / 4; ++g)
    hi[g] = fp8x4(ldexpf(v[4 * g], -eh), ldexpf(v[4 * g + 1], -eh), ldexpf(v[4 * g + 2], -eh),
                  ldexpf(v[4 * g + 3], -eh));
  float r[N];
#pragma unroll
  for (int g = 0; g < N / 4; ++g) {
    r[4 * g + 0] = v[4 * g + 0] - ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)hi[g], 0), eh);
    r[4 * g + 1] = v[4 * g + 1] - ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)hi[g], 1), eh);
    r[4 * g + 2] = v[4 * g + 2] - ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)hi[g], 2), eh);
    r[4 * g + 3] = v[4 * g + 3] - ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)hi[g], 3), eh);
  }
  float mr = 0.f;
#pragma unroll
  for (int j = 0; j < N; ++j) mr = fmaxf(mr, fabsf(r[j]));
  if (PARTNER) mr = fmaxf(mr, __shfl_xor(mr, 16));
  el = mx8_exp(mr);
#pragma unroll
  for (int g = 0; g < N / 4; ++g)
    lo[g] = fp8x4(ldexpf(r[4 * g], -el), ldexpf(r[4 * g + 1], -el), ldexpf(r[4 * g + 2], -el),
                  ldexpf(r[4 * g + 3], -el));
}
// Four values per lane; the block is the 32 values of an aligned 8-lane group (the maxima by DPP
// steps on the magnitudes' bit patterns, which order like the magnitudes). The same hi and lo
// words and exponents as mx8_quant over those 32 values.
__device__ __forceinline__ void mx8_quant4_g8(const float (&v)[4], uint32_t& hi, uint32_t& lo, int& eh, int& el) {
  auto gmax8 = [](uint32_t m) {
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
    return max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xf, 0xf, false));  // row_half_mirror
  };
  uint32_t m = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) m = max(m, __float_as_uint(fabsf(v[j])));
  eh = mx8_exp(__uint_as_float(gmax8(m)));
  hi = fp8x4(ldexpf(v[0], -eh), ldexpf(v[1], -eh), ldexpf(v[2], -eh), ldexpf(v[3], -eh));
  float r[4];
  r[0] = v[0] - ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)hi, 0), eh);
  r[1] = v[1] - ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)hi, 1), eh);
  r[2] = v[2] - ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)hi, 2), eh);
  r[3] = v[3] - ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)hi, 3), eh);
  uint32_t mr = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) mr = max(mr, __float_as_uint(fabsf(r[j])));
  el = mx8_exp(__uint_as_float(gmax8(mr)));
  lo = fp8x4(ldexpf(r[0], -el), ldexpf(r[1], -el), ldexpf(r[2], -el), ldexpf(r[3], -el));
}
// MXW window layout: the 16 values of (column c, 32-block blk, half h) sit as bytes L 32 + off ..
// + 15 of the hi part (bytes 2048 + the same of the lo part), L = c + 16 (2 (blk mod 2) + h),
// off = 16 (blk / 2), value j of the half in byte j; the block's scale pair (hi exponent + 127 in
// byte 0, lo in byte 1) is the word at 4096 + 4 (c + 16 blk).
__device__ __forceinline__ f32x4 mfma_mx(u32x4 a, uint32_t sa, u32x4 b0, u32x4 b1, uint32_t sb, int sel, f32x4 acc) {
  const v8i A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  if (sel == 0) return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 4, 0, 0, (int)sa, 0, (int)sb);
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 4, 0, 0, (int)sa, 1, (int)sb);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Offset (in values) of lane quad q, k-step j inside a 128-wide window.
__device__ __forceinline__ int kofs(int j, int q) { return 32 * j + 8 * q; }

// (value, index) maximum with equal values going to the lower index.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    float ov = __shfl_xor(v, off);
    int oi = __shfl_xor(i, off);
    argmax_merge(v, i, ov, oi);
  }
}

struct Args {
  const float* x;
  float* y;
  int32_t* out_ids;
  float* out_w;
  int32_t* out_n;
  const float* wr;
  const uint8_t* wg;
  const uint8_t* wu;
  const uint8_t* wd;
  const uint8_t* sg;
  const uint8_t* su;
  const uint8_t* sd;
  const uint8_t* shg;
  const uint8_t* shu;
  const uint8_t* shd;
  int32_t* tab_n;     // U
  uint32_t* ctr;      // [2][NGRP] pool counters of the gate/up and down kernels, CTR_STRIDE words
                      // apart (zeroed by the router)
  int32_t* tab_woken; // [umax] woken expert ids, ascending
  int8_t* tab_slot;   // [umax][16] slot of token t for woken expert u, or -1
  u32x4* xfrag;   // the block's B operands: bf16 layers (H/32) k-steps x {hi, lo} x 64 lanes;
                  // mxfp4 layers (H/128) MX-fp8 windows of MXW bytes
  u32x4* xfrag_sh;   // bf16 hi/lo fragments for the shared expert of mxfp4 layers
  float* plog;    // [hs][16][E] partial raw logits
  float* psq;     // [hs][16] partial sums of squares
  u32x4* afrag;   // [umax][(I/32) x {hi, lo} x 64 lanes]
  u32x4* afrag_sh;
  float* part;    // [k][K+1][H]
  int H, E, K, I, Is, k, hs, ntile_e, umax, pre_norm, residual;
  float eps;
};

struct alignas(16) Smem {
  float red[16384];           // per-wave partial tiles (gate/up, down)
  float act[GU_MX_RT][256];   // reduced, activated gate/up tiles
  int ids[KMAX][MAX_K];
  float w[KMAX][MAX_K];
  uint8_t flag[MAX_E];
  int pos[MAX_E];
  int woken[MAX_U];
  float wcol[MAX_U + 1][KMAX];
  alignas(8) int8_t slot[MAX_U][KMAX];
  float rinv[KMAX];
  int nw;
  int claim[4];  // ring of claimed item indices: item n sits in claim[n % 4]
};

// ------------------------------------------------------------------------------------------
// router item (expert tile, H slice) with fp32 MFMA 16x16x4
// ------------------------------------------------------------------------------------------
// k-step s of the block as bf16 hi/lo MFMA B fragments
__device__ __forceinline__ void write_xfrag(const float* x, u32x4* dst, int H, int k, int s, int lane) {
  const int t = lane & 15, qq = lane >> 4, w = s >> 2, j = s & 3;
  uint32_t hi[8], lo[8];
  if (t < k) {
    const float* src = x + (size_t)t * H + w * WIN + kofs(j, qq);
    const float4 v0 = *reinterpret_cast<const float4*>(src);
    const float4 v1 = *reinterpret_cast<const float4*>(src + 4);
    const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) split_bf16(f[i], hi[i], lo[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) hi[i] = lo[i] = 0u;
  }
  u32x4 h, l;
  pack8(hi, h);
  pack8(lo, l);
  dst[((size_t)s * 2 + 0) * 64 + lane] = h;
  dst[((size_t)s * 2 + 1) * 64 + lane] = l;
}

// window w of the raw block as MX-fp8 hi + lo B fragments with their scales (mxfp4 layers), by a
// whole workgroup: thread (token c, 32-block b, group g) quantises values 4 g .. 4 g + 3 of block b
// of token c, the eight threads of an aligned 8-lane group sharing the block maximum, and stores
// them where the instruction's B layout puts them (one lane per block did the 32 values before)
__device__ __forceinline__ void write_xmx(const float* x, uint8_t* dst, int H, int k, int w, int tid) {
  const int c = tid >> 5, b = (tid >> 3) & 3, g = tid & 7;
  const float4 f = *reinterpret_cast<const float4*>(x + (size_t)(c < k ? c : 0) * H + w * WIN + 32 * b + 4 * g);
  const float v[4] = {c < k ? f.x : 0.f, c < k ? f.y : 0.f, c < k ? f.z : 0.f, c < k ? f.w : 0.f};
  uint32_t hi, lo;
  int eh, el;
  mx8_quant4_g8(v, hi, lo, eh, el);
  uint8_t* win = dst + (size_t)w * MXW;
  const int h = g >> 2, q = g & 3;
  const int L = c + 16 * (2 * (b & 1) + h), off = 16 * (b >> 1) + 4 * q;  // the MXW window layout
  *reinterpret_cast<uint32_t*>(win + L * 32 + off) = hi;
  *reinterpret_cast<uint32_t*>(win + 2048 + L * 32 + off) = lo;
  if (g == 0)
    *reinterpret_cast<uint32_t*>(win + 4096 + (c + 16 * b) * 4) = (uint32_t)(eh + 127) | ((uint32_t)(el + 127) << 8);
}

struct RouterSmem {
  float red[NW * 256];
  float rsq[NW][64];
};

template <bool MX>
__device__ void router_item(const Args& a, RouterSmem& S, int r, int wave, int lane, int tid) {
  const int H = a.H, E = a.E, k = a.k;
  const int tile = r % a.ntile_e, hsi = r / a.ntile_e;
  const int cpw = H / (a.hs * NW);  // columns per wave, a multiple of 16
  const int c0 = hsi * (H / a.hs) + wave * cpw;
  const int row = lane & 15, q = lane >> 4;
  const int e = tile * 16 + row;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  const float* wrow = a.wr + (size_t)(e < E ? e : 0) * H;
  const float* xrow = a.x + (size_t)(row < k ? row : 0) * H;
  for (int m = 0; m < cpw / 16; ++m) {
    const int h = c0 + 16 * m + 4 * q;
    float4 wv = *reinterpret_cast<const float4*>(wrow + h);
    float4 xv = *reinterpret_cast<const float4*>(xrow + h);
    if (e >= E) wv = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row >= k) xv = make_float4(0.f, 0.f, 0.f, 0.f);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wv.x, xv.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wv.y, xv.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wv.z, xv.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wv.w, xv.w, acc, 0, 0, 0);
    ss += xv.x * xv.x + xv.y * xv.y + xv.z * xv.z + xv.w * xv.w;
  }
  *reinterpret_cast<f32x4*>(&S.red[wave * 256 + lane * 4]) = acc;
  S.rsq[wave][lane] = ss;
  __syncthreads();
  if (tid < 256) {
    // D[i][j]: lane j + 16 (i / 4), element i % 4; i = expert within the tile, j = token
    float d = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) d += S.red[w * 256 + tid];
    const int l = tid >> 2, v = tid & 3;
    const int t = l & 15, ei = tile * 16 + 4 * (l >> 4) + v;
    if (t < k && ei < E) a.plog[((size_t)hsi * KMAX + t) * E + ei] = d;
  }
  if (tile == 0 && tid < KMAX) {
    float s = 0.f;
    for (int w = 0; w < NW; ++w)
      for (int qq = 0; qq < 4; ++qq) s += S.rsq[w][tid + 16 * qq];
    a.psq[hsi * KMAX + tid] = s;
  }
  // B-operand fragments of the raw block, spread over the router's waves: bf16 hi/lo k-steps
  // (bf16 layers, and the shared expert of mxfp4 layers), MX-fp8 windows (mxfp4 routed experts)
  const int nr = a.ntile_e * a.hs;
  if (!MX) {
    for (int s = r + nr * (tid >> 6); s < H / 32; s += nr * NW) write_xfrag(a.x, a.xfrag, H, k, s, lane);
  } else {
    static_assert(NTH == 16 * 4 * 8, "one workgroup per MX-fp8 window");
    for (int w = r; w < H / WIN; w += nr) write_xmx(a.x, reinterpret_cast<uint8_t*>(a.xfrag), H, k, w, tid);
    if (a.Is > 0)
      for (int s = r + nr * (tid >> 6); s < H / 32; s += nr * NW) write_xfrag(a.x, a.xfrag_sh, H, k, s, lane);
  }
}

// Order-preserving 32-bit key of a logit: a larger logit has a larger key; -0 counts as +0; NaN
// maps to 1, below every number; 0 marks an empty or already-picked slot.
__device__ __forceinline__ uint32_t okey32(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return v != v ? 1u : k;
}
__device__ __forceinline__ float okey32_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}
// Wave-wide maximum / minimum of a 32-bit value in every lane: DPP steps inside 16-lane rows, then
// the gfx950 row and half swaps (no LDS round trips, unlike lane shuffles).
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
  x = op(x, dpp_u32<0xB1>(x));   // quad_perm [1,0,3,2]
  x = op(x, dpp_u32<0x4E>(x));   // quad_perm [2,3,0,1]
  x = op(x, dpp_u32<0x141>(x));  // row_half_mirror
  x = op(x, dpp_u32<0x140>(x));  // row_mirror
  const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op((uint32_t)r16[0], (uint32_t)r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op((uint32_t)r32[0], (uint32_t)r32[1]);
}
// The same maximum over each 16-lane row of the wave (DPP steps that stay inside a row), in every
// lane of the row.
__device__ __forceinline__ void row16_argmax_dpp(float& v, int& i) {
  auto red = [](uint32_t x, bool mx) {
    auto op = [mx](uint32_t a, uint32_t b) { return mx ? max(a, b) : min(a, b); };
    x = op(x, dpp_u32<0xB1>(x));   // quad_perm [1,0,3,2]
    x = op(x, dpp_u32<0x4E>(x));   // quad_perm [2,3,0,1]
    x = op(x, dpp_u32<0x141>(x));  // row_half_mirror
    return op(x, dpp_u32<0x140>(x));  // row_mirror
  };
  const uint32_t key = okey32(v);
  const uint32_t km = red(key, true);
  const uint32_t im = red(key == km ? (uint32_t)i : 0xFFFFFFFFu, false);
  v = km == 1u ? v : okey32_value(km);  // a row of NaNs keeps its own value
  i = (int)im;
}
// (value, index) maximum over the wave, equal values to the lower index, in every lane: the
// largest order-preserving key, then the lowest index among the lanes holding it. The same
// result as merging the lanes with argmax_merge (-0 and +0 are equal; a NaN never wins over a
// number), with the value returned as the key's float (+0 for a -0 maximum).
__device__ __forceinline__ void wave_argmax_dpp(float& v, int& i) {
  const uint32_t key = okey32(v);
  const uint32_t km = wave_reduce_u32<true>(key);
  const uint32_t im = wave_reduce_u32<false>(key == km ? (uint32_t)i : 0xFFFFFFFFu);
  v = km == 1u ? v : okey32_value(km);  // a wave of NaNs keeps its own value
  i = (int)im;
}

// Top-K candidates are (key, expert) composites: the order-preserving logit key in the upper word
// and the inverted expert id in the lower, so the larger composite is the larger logit and, on
// equal logits, the lower expert id. Experts are laid out lane-major (lane l holds experts
// NS l .. NS l + NS - 1), so among lanes whose heads tie, the lowest lane holds the lowest id.
__device__ __forceinline__ uint64_t topk_comp(uint32_t key, int e) {
  return ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)e);
}
__device__ __forceinline__ void cmpx(uint64_t& a, uint64_t& b) {  // a takes the larger
  const bool s = b > a;
  const uint64_t t = s ? b : a;
  b = s ? a : b;
  a = t;
}
// descending sort of a lane's candidates: the 5- and 19-comparator networks for 4 and 8 inputs
template <int NS>
__device__ __forceinline__ void sort_desc(uint64_t (&c)[NS]) {
  static_assert(NS == 4 || NS == 8, "4 or 8 candidates per lane");
  if constexpr (NS == 4) {
    cmpx(c[0], c[1]); cmpx(c[2], c[3]); cmpx(c[0], c[2]); cmpx(c[1], c[3]); cmpx(c[1], c[2]);
  } else {
    cmpx(c[0], c[1]); cmpx(c[2], c[3]); cmpx(c[4], c[5]); cmpx(c[6], c[7]);
    cmpx(c[0], c[2]); cmpx(c[1], c[3]); cmpx(c[4], c[6]); cmpx(c[5], c[7]);
    cmpx(c[1], c[2]); cmpx(c[5], c[6]);
    cmpx(c[0], c[4]); cmpx(c[1], c[5]); cmpx(c[2], c[6]); cmpx(c[3], c[7]);
    cmpx(c[2], c[4]); cmpx(c[3], c[5]);
    cmpx(c[1], c[2]); cmpx(c[3], c[4]); cmpx(c[5], c[6]);
  }
}

// K rounds over the lanes' sorted candidate lists: each round takes the maximum of the list
// heads (DPP steps inside 16-lane rows, then a row swap that pairs rows 0-1 and 2-3, and for a
// whole wave a half swap, so the maximum sits in a VGPR of every lane), the lowest lane whose head
// equals it (one ballot) and pops that lane's head. HALF: the wave serves two tokens, lanes 0-31
// and 32-63; no step crosses a half, so each half picks its own token's next expert. Lane j of a
// half records pick j (expert and key).
// The sorted list is split into its 32-bit keys and the candidates' positions m inside the lane
// (4 bits each, head in the low bits): the expert of the winning head is NS (lane - first lane of
// the half) + m, so a pop shifts NS keys and one word instead of NS 64-bit composites.
template <int NS, bool HALF>
__device__ __forceinline__ void topk_sorted(const uint64_t (&c)[NS], int K, int lane, int& my_e, uint32_t& my_key) {
  static_assert(NS <= 8, "4-bit positions, 8 per word");
  const bool hi = HALF && lane >= 32;
  const int jl = HALF ? (lane & 31) : lane;
  uint32_t kk[NS];
  uint32_t pk = 0;
#pragma unroll
  for (int m = 0; m < NS; ++m) {
    kk[m] = (uint32_t)(c[m] >> 32);
    pk |= ((~(uint32_t)c[m]) & (uint32_t)(NS - 1)) << (4 * m);  // expert NS l + position
  }
  for (int j = 0; j < K; ++j) {
    const uint32_t h = kk[0];
    uint32_t x = h;
    x = max(x, dpp_u32<0xB1>(x));   // quad_perm [1,0,3,2]
    x = max(x, dpp_u32<0x4E>(x));   // quad_perm [2,3,0,1]
    x = max(x, dpp_u32<0x141>(x));  // row_half_mirror
    x = max(x, dpp_u32<0x140>(x));  // row_mirror: the row maximum in every lane of the row
    // v_permlane16_swap: one copy gets rows (0, 0, 2, 2), the other rows (1, 1, 3, 3)
    const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    uint32_t w = max((uint32_t)r16[0], (uint32_t)r16[1]);  // the half's maximum
    if constexpr (!HALF) {  // v_permlane32_swap: halves (0, 0) and (1, 1)
      const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
      w = max((uint32_t)r32[0], (uint32_t)r32[1]);
    }
    int e, sl;
    if constexpr (HALF) {
      const uint64_t bm = __ballot(h == w);  // each half holds its own maximum
      const int sla = __builtin_ctz((uint32_t)bm), slb = 32 + __builtin_ctz((uint32_t)(bm >> 32));
      const int ea = NS * sla + (int)((uint32_t)__builtin_amdgcn_readlane((int)pk, sla) & 15u);
      const int eb = NS * (slb - 32) + (int)((uint32_t)__builtin_amdgcn_readlane((int)pk, slb) & 15u);
      sl = hi ? slb : sla;
      e = hi ? eb : ea;
    } else {
      sl = __builtin_ctzll(__ballot(h == w));
      e = NS * sl + (int)((uint32_t)__builtin_amdgcn_readlane((int)pk, sl) & 15u);
    }
    if (jl == j) { my_e = e; my_key = w; }
    // the pop as bit selects under an all-ones / zero mask that the optimizer cannot see through:
    // written as selects on the lane test, the shifts were turned into per-key position tracking
    // with compare chains, three times the instructions
    uint32_t pm = lane == sl ? ~0u : 0u;
    asm volatile("" : "+v"(pm));
#pragma unroll
    for (int m = 0; m + 1 < NS; ++m) kk[m] = (kk[m] & ~pm) | (kk[m + 1] & pm);
    kk[NS - 1] &= ~pm;
    pk = (pk & ~pm) | ((pk >> 4) & pm);
  }
}

// A lane's NS consecutive logits row[e0 .. e0 + NS - 1] of one token (LDS or global; values past
// E are read at E - 1 and masked by the caller): float4 reads when E is a multiple of 4 and the
// lane's run lies inside the row (row starts are then 16-byte aligned), else clamped scalar
// reads; all issued before any is used.
template <int NS>
__device__ __forceinline__ void lane_logits(const float* row, int e0, int E, float (&v)[NS]) {
  if (E % 4 == 0 && e0 + NS <= E) {
#pragma unroll
    for (int m = 0; m < NS; m += 4) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(row + e0 + m);
      v[m] = q[0]; v[m + 1] = q[1]; v[m + 2] = q[2]; v[m + 3] = q[3];
    }
  } else {
#pragma unroll
    for (int m = 0; m < NS; ++m) v[m] = row[min(e0 + m, E - 1)];
  }
}

// ------------------------------------------------------------------------------------------
// routing (every gate/up workgroup, into LDS)
// ------------------------------------------------------------------------------------------
// The router's H-slice partials of the block, requested before anything else the gate/up kernel
// loads. Vector-memory results return in issue order, so a workgroup that then requests its
// shared-expert tile still sums the partials without waiting for that tile. When E is a multiple
// of 4 a thread loads float4s of (token, 4 experts, slice), at most 16 loads (4 pairs x 4 slices);
// 64 scalar loads per thread would exceed the 63 loads one wave can have outstanding and cost a
// second round trip. Addresses are clamped into the slab; the results are used only in route()
// (selected there), so nothing waits on them before the shared tile is requested.
struct RoutePart {
  f32x4 v[4][HS_MAX];  // (pair i: token, expert quad) x slice; pair P = tid + NTH i
  float q[HS_MAX];     // sums of squares of token tid (tid < KMAX)
};
__device__ __forceinline__ RoutePart route_issue(const Args& a, int tid) {
  RoutePart r;
  const int E = a.E, hs = a.hs, k = a.k;
  // buffer loads: one 32-bit lane offset per pair, the slice offset in an SGPR
  const rsrc_t rl = buf_rsrc(a.plog, (uint32_t)(hs * KMAX * E * 4));
  const rsrc_t rq = buf_rsrc(a.psq, (uint32_t)(hs * KMAX * 4));
  if (E % 4 == 0) {
    const int nq = E >> 2, np = KMAX * nq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int P = tid + NTH * i;
      const int Pc = P < np ? P : 0, t = Pc / nq, q = Pc % nq;
      const uint32_t vo = (uint32_t)(((t < k ? t : 0) * E + 4 * q) * 4);
#pragma unroll
      for (int h = 0; h < HS_MAX; ++h)
        r.v[i][h] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rl, vo, (uint32_t)((h < hs ? h : 0) * KMAX * E * 4), 0));
    }
  }
  const uint32_t vq = (uint32_t)((tid < KMAX ? tid : 0) * 4);
#pragma unroll
  for (int h = 0; h < HS_MAX; ++h)
    r.q[h] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rq, vq, (uint32_t)((h < hs ? h : 0) * KMAX * 4), 0));
  return r;
}

__device__ void route(const Args& a, Smem& S, RoutePart rp, int wave, int lane, int tid) {
  const int E = a.E, K = a.K, k = a.k, hs = a.hs;
  // The partials are opaque to the optimizer from here on (an empty asm that reads and writes
  // their registers), so no arithmetic on them is hoisted above the caller's later loads; such an
  // add made the wave wait for the partials before the shared tile was requested.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < HS_MAX; ++h) asm volatile("" : "+v"(rp.v[i][h]));
#pragma unroll
  for (int h = 0; h < HS_MAX; ++h) asm volatile("" : "+v"(rp.q[h]));
  // Sum the router's H-slice partials into S.red[t * E + e] (slices in ascending order).
  float* lg = S.red;
  if (E % 4 == 0) {
    const int nq = E >> 2, np = KMAX * nq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int P = tid + NTH * i, t = P / nq, q = P % nq;
      f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < HS_MAX; ++h) sum = h < hs ? sum + rp.v[i][h] : sum;
      if (P < np && t < k) *reinterpret_cast<f32x4*>(&lg[t * E + 4 * q]) = sum;
    }
  } else {  // thread e loads all of expert e's partials at once, then sums them
    const int e = tid < E ? tid : 0;
    float p[KMAX][HS_MAX];
#pragma unroll
    for (int t = 0; t < KMAX; ++t)
#pragma unroll
      for (int h = 0; h < HS_MAX; ++h)
        p[t][h] = a.plog[((size_t)(h < hs ? h : 0) * KMAX + (t < k ? t : 0)) * E + e];
#pragma unroll
    for (int t = 0; t < KMAX; ++t) {
      float sum = 0.f;
#pragma unroll
      for (int h = 0; h < HS_MAX; ++h) sum = h < hs ? sum + p[t][h] : sum;
      if (t < k && tid < E) lg[t * E + tid] = sum;
    }
  }
  if (tid < KMAX) {
    float ssq = 0.f;
#pragma unroll
    for (int h = 0; h < HS_MAX; ++h) ssq = h < hs ? ssq + rp.q[h] : ssq;
    S.rinv[tid] = a.pre_norm ? 1.0f / sqrtf(ssq / (float)a.H + a.eps) : 1.0f;
  }
  for (int i = tid; i < MAX_E; i += NTH) S.flag[i] = 0;
  {  // the weight table (umax routed rows and the shared row) and the slot table start empty
    float* wc = &S.wcol[0][0];
    for (int i = tid; i < (a.umax + 1) * KMAX; i += NTH) wc[i] = 0.f;
    uint32_t* sl = reinterpret_cast<uint32_t*>(&S.slot[0][0]);
    for (int i = tid; i < a.umax * KMAX / 4; i += NTH) sl[i] = 0xFFFFFFFFu;  // every byte -1
  }
  __syncthreads();
  // Top-K per token (wave w serves tokens w and w + 8), then the softmax over the K in the same
  // wave. Ties go to the lower expert id.
  static_assert(MAX_E == 8 * 64 && KMAX == 2 * NW, "top-K layout");
  if (E <= 256 && k > NW) {
    // both tokens at once, half a wave each, 8 candidates per lane (expert 8 (lane mod 32) + m)
    const int t = wave + (lane >= 32 ? NW : 0);
    const bool live = t < k;
    const float rv = S.rinv[live ? t : wave];
    const int e0 = 8 * (lane & 31);
    float v[8];
    lane_logits<8>(lg + t * E, e0, E, v);  // rows past k are in bounds, unused
    uint64_t c[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int e = e0 + m;
      c[m] = topk_comp((live && e < E) ? okey32(rv * v[m]) : 0u, e);
    }
    sort_desc<8>(c);
    int my_e = 0;
    uint32_t my_key = 0;
    topk_sorted<8, true>(c, K, lane, my_e, my_key);
    const float my_val = okey32_value(my_key);
    const int base = lane & 32;  // first lane of this half
    const float m0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_val), 0));
    const float m1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_val), 32));
    const float ex = expf(my_val - (base ? m1 : m0));
    float sa = 0.f, sb = 0.f;
    for (int j = 0; j < K; ++j) {
      sa += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
      sb += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), 32 + j));
    }
    const int j = lane & 31;
    if (live && j < K) {
      S.ids[t][j] = my_e;
      S.w[t][j] = ex / (base ? sb : sa);
      S.flag[my_e] = 1;
    }
  } else {
    for (int t = wave; t < k; t += NW) {
      const float rv = S.rinv[t];
      int my_e = 0;
      uint32_t my_key = 0;
      if (E <= 256) {  // 4 candidates per lane: experts 4 lane + m
        float v[4];
        lane_logits<4>(lg + t * E, 4 * lane, E, v);
        uint64_t c[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int e = 4 * lane + m;
          c[m] = topk_comp(e < E ? okey32(rv * v[m]) : 0u, e);
        }
        sort_desc<4>(c);
        topk_sorted<4, false>(c, K, lane, my_e, my_key);
      } else {  // 8 candidates per lane: experts 8 lane + m
        float v[8];
        lane_logits<8>(lg + t * E, 8 * lane, E, v);
        uint64_t c[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int e = 8 * lane + m;
          c[m] = topk_comp(e < E ? okey32(rv * v[m]) : 0u, e);
        }
        sort_desc<8>(c);
        topk_sorted<8, false>(c, K, lane, my_e, my_key);
      }
      const float my_val = okey32_value(my_key);
      const float m0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_val), 0));
      const float ex = expf(my_val - m0);
      float sum = 0.f;
      for (int j = 0; j < K; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
      if (lane < K) {
        S.ids[t][lane] = my_e;
        S.w[t][lane] = ex / sum;
        S.flag[my_e] = 1;
      }
    }
  }
  __syncthreads();
  if (wave == 0) {  // the union in ascending expert order: all flags read at once, then ballots
    bool f[MAX_E / 64];
#pragma unroll
    for (int c = 0; c < MAX_E / 64; ++c) f[c] = S.flag[c * 64 + lane] != 0;  // zero past E
    int base = 0;
#pragma unroll
    for (int c = 0; c < MAX_E / 64; ++c) {
      const int e = c * 64 + lane;
      const unsigned long long m = __ballot(f[c]);
      const int p = base + __popcll(m & ((1ull << lane) - 1ull));
      if (f[c]) { S.woken[p] = e; S.pos[e] = p; }
      base += __popcll(m);
    }
    if (lane == 0) S.nw = base;
  }
  __syncthreads();
  const int U = S.nw;
  if (tid < k * K) {
    const int t = tid / K, j = tid % K;
    const int u = S.pos[S.ids[t][j]];
    S.wcol[u][t] = S.w[t][j];
    S.slot[u][t] = (int8_t)j;
  }
  if (tid < KMAX) S.wcol[U][tid] = (tid < k) ? 1.0f : 0.f;  // shared expert column weights
  __syncthreads();
  if (blockIdx.x == 0) {  // outputs
    if (tid < k * K) {
      const int t = tid / K, j = tid % K;
      if (a.out_ids) a.out_ids[t * K + j] = S.ids[t][j];
      if (a.out_w) a.out_w[t * K + j] = S.w[t][j];
    }
    // written through to memory, like a later failure report (-1) that must not be overwritten
    if (tid == 0 && a.out_n) st_dev(reinterpret_cast<uint32_t*>(a.out_n), (uint32_t)U);
  }
}

// ------------------------------------------------------------------------------------------
// gate/up items. Wave w owns H-windows w*WPW .. w*WPW+WPW-1.
// ------------------------------------------------------------------------------------------
template <int WPW>
struct GUItem {
  u32x4 v[WPW * 8];                // bf16: [(wi*2 + mat)*4 + j]; mxfp4: [(tile*WPW + wi)*2 + mat]
  uint32_t sc[GU_MX_RT * WPW * 2];
};

struct GUDesc {
  int u, row0, ntile;
  uint32_t off;   // byte offset of the item in the gate / up tensors (codes for mxfp4)
  uint32_t soff;  // byte offset of the item's scales (mxfp4)
};

// buffer resources of the gate/up kernel's weight streams
struct GURes {
  rsrc_t g, u, sg, su;
};

// bf16 item (one 16-row tile of g / up, tiled layout): lane reads its 16 B of each 1 KiB
// fragment tile; the four k-steps of a window are 4 KiB contiguous.
template <int WPW>
__device__ __forceinline__ void gu_load_bf16(GUItem<WPW>& T, rsrc_t rg, rsrc_t ru, uint32_t soff, uint32_t vb) {
#pragma unroll
  for (int wi = 0; wi < WPW; ++wi)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t o = vb + (uint32_t)((4 * wi + j) * 1024);
      T.v[(wi * 2 + 0) * 4 + j] = bld16(rg, o, soff);
      T.v[(wi * 2 + 1) * 4 + j] = bld16(ru, o, soff);
    }
}

// mxfp4 item (GU_MX_RT tiles of 16 rows, tiled layout): per (tile, window) the codes are 1 KiB
// contiguous (lane = one 32-value block) and the scales 64 B contiguous.
template <int WPW>
__device__ __forceinline__ void gu_load_mx(GUItem<WPW>& T, const GURes& R, const GUDesc& d, int H, uint32_t vbc,
                                           uint32_t vbs) {
#pragma unroll
  for (int tl = 0; tl < GU_MX_RT; ++tl)
#pragma unroll
    for (int wi = 0; wi < WPW; ++wi) {
      const uint32_t sc = d.off + (uint32_t)(16 * tl * (H / 2)), ss = d.soff + (uint32_t)(16 * tl * (H / 32));
      T.v[(tl * WPW + wi) * 2 + 0] = bld16(R.g, vbc + wi * 1024, sc);
      T.v[(tl * WPW + wi) * 2 + 1] = bld16(R.u, vbc + wi * 1024, sc);
      T.sc[(tl * WPW + wi) * 2 + 0] = bld1(R.sg, vbs + wi * 64, ss);
      T.sc[(tl * WPW + wi) * 2 + 1] = bld1(R.su, vbs + wi * 64, ss);
    }
}

// Cross-wave reduction, SwiGLU with the RMSNorm factor and the routing weight, hi/lo split, and
// the store as down-projection B fragments (rows row0 .. row0 + 16 ntile of expert slot `u`):
// bf16 hi/lo fragments, or (MX8: routed items of mxfp4 layers, 32 rows = one 32-value block of
// the down projection's reduction dimension) MX-fp8 hi/lo operands with their block scales.
template <bool MX8 = false>
__device__ __forceinline__ void gu_epilogue(const Args& a, Smem& S, const f32x4 (&acc)[GU_MX_RT][2],
                                            int ntile, int u, int row0, bool routed, int wave,
                                            int lane, int tid, int ring = -1, int* next = nullptr) {
#pragma unroll
  for (int tl = 0; tl < GU_MX_RT; ++tl)
    if (tl < ntile) {
      *reinterpret_cast<f32x4*>(&S.red[((wave * GU_MX_RT + tl) * 2 + 0) * 256 + lane * 4]) = acc[tl][0];
      *reinterpret_cast<f32x4*>(&S.red[((wave * GU_MX_RT + tl) * 2 + 1) * 256 + lane * 4]) = acc[tl][1];
    }
  __syncthreads();
  for (int i = tid; i < ntile * 256; i += NTH) {
    const int tl = i >> 8, p = i & 255;
    float g = 0.f, up = 0.f;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) {
      g += S.red[((wv * GU_MX_RT + tl) * 2 + 0) * 256 + p];
      up += S.red[((wv * GU_MX_RT + tl) * 2 + 1) * 256 + p];
    }
    const int c = (p >> 2) & 15;
    const float rv = S.rinv[c];
    S.act[tl][p] = silu(g * rv) * (up * rv) * S.wcol[u][c];
  }
  __syncthreads();
  if (ring >= 0) {  // the next item index, read before this epilogue's stores are issued
    *next = __builtin_amdgcn_readfirstlane(S.claim[ring]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (MX8) {
    // thread (block bb, column c, group g) -> rows 32 bb + 4 g .. + 3 of the item: eight threads
    // of one aligned 8-lane group share a column's 32-row block (two waves per block; the
    // quantisation took one half-wave per block before, 1.7 us of a k = 16 call)
    if (tid < 64 * ntile) {
      const int g = tid & 7, c = (tid >> 3) & 15, bb = tid >> 7, h = g >> 2, q = g & 3;
      const f32x4 x4 = *reinterpret_cast<const f32x4*>(&S.act[2 * bb + h][(c + 16 * q) * 4]);
      const float v[4] = {x4[0], x4[1], x4[2], x4[3]};
      uint32_t hi, lo;
      int eh, el;
      mx8_quant4_g8(v, hi, lo, eh, el);
      uint8_t* win = reinterpret_cast<uint8_t*>(a.afrag) + ((size_t)u * (a.I / WIN) + row0 / WIN) * MXW;
      const int blk = (row0 % WIN) / 32 + bb;
      const int L = c + 16 * (2 * (blk & 1) + h), off = 16 * (blk >> 1) + 4 * q;  // the MXW window layout
      const uint32_t sw = (uint32_t)(eh + 127) | ((uint32_t)(el + 127) << 8);
      st_dev(reinterpret_cast<uint32_t*>(win + L * 32 + off), hi);  // published inside the launch
      st_dev(reinterpret_cast<uint32_t*>(win + 2048 + L * 32 + off), lo);
      if (g == 0) st_dev(reinterpret_cast<uint32_t*>(win + 4096 + (c + 16 * blk) * 4), sw);
    }
    return;
  }
  // thread (tile, half, column c, pair m) -> rows R + 2 m and R + 2 m + 1 of the expert's
  // intermediate dimension, R = row0 + 16 tile + 8 half: word m of the 16-byte hi and lo
  // fragments that hold rows R .. R + 7 of column c (128 threads per tile; the split took 32
  // threads with eight rows each before)
  if (tid < ntile * 2 * KMAX * 4) {
    const int m = tid & 3, c = (tid >> 2) & 15, half = (tid >> 6) & 1, tl = tid >> 7;
    const int r = half * 8 + 2 * m;  // rows r and r + 1 sit side by side in the act tile
    const float2 v = *reinterpret_cast<const float2*>(&S.act[tl][(c + 16 * (r >> 2)) * 4 + (r & 3)]);
    uint32_t h0, l0, h1, l1;
    split_bf16(v.x, h0, l0);
    split_bf16(v.y, h1, l1);
    const int R = row0 + 16 * tl + 8 * half;
    const int w = R / WIN, o = R % WIN;
    const int j = o / 32, q = (o % 32) / 8;
    const int s = w * 4 + j;
    const int I = routed ? a.I : a.Is;
    u32x4* dst = routed ? a.afrag + (size_t)u * (I / 32) * 128 : a.afrag_sh;
    uint32_t* ph = reinterpret_cast<uint32_t*>(dst + ((size_t)s * 2 + 0) * 64 + c + 16 * q) + m;
    uint32_t* pl = reinterpret_cast<uint32_t*>(dst + ((size_t)s * 2 + 1) * 64 + c + 16 * q) + m;
    st_dev(ph, h0 | (h1 << 16));  // published inside the launch
    st_dev(pl, l0 | (l1 << 16));
  }
}

template <int WPW>
__device__ __forceinline__ void gu_math_bf16(f32x4 (&acc)[GU_MX_RT][2], const GUItem<WPW>& T,
                                             const u32x4 (&xb)[WPW][4][2]) {
#pragma unroll
  for (int tl = 0; tl < GU_MX_RT; ++tl) acc[tl][0] = acc[tl][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int wi = 0; wi < WPW; ++wi)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int mat = 0; mat < 2; ++mat) {
        acc[0][mat] = mfma16(T.v[(wi * 2 + mat) * 4 + j], xb[wi][j][0], acc[0][mat]);
        acc[0][mat] = mfma16(T.v[(wi * 2 + mat) * 4 + j], xb[wi][j][1], acc[0][mat]);
      }
}

// MX-fp8 B operands of this wave's H windows (mxfp4 routed experts): hi and lo halves, scales
template <int WPW>
struct XMX {
  u32x4 hi[WPW][2], lo[WPW][2];
  uint32_t sc[WPW];
};
template <int WPW>
__device__ __forceinline__ void gu_load_xmx(XMX<WPW>& xm, const u32x4* xf, int win0, bool active, int lane) {
  const uint8_t* base = reinterpret_cast<const uint8_t*>(xf);
#pragma unroll
  for (int wi = 0; wi < WPW; ++wi) {
    const uint8_t* w = base + (size_t)(active ? win0 + wi : 0) * MXW;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const u32x4 h = *reinterpret_cast<const u32x4*>(w + lane * 32 + 16 * hh);
      const u32x4 l = *reinterpret_cast<const u32x4*>(w + 2048 + lane * 32 + 16 * hh);
      xm.hi[wi][hh] = active ? h : u32x4{0u, 0u, 0u, 0u};  // inactive waves multiply by zero
      xm.lo[wi][hh] = active ? l : u32x4{0u, 0u, 0u, 0u};
    }
    xm.sc[wi] = *reinterpret_cast<const uint32_t*>(w + 4096 + lane * 4);
  }
}

// mxfp4 item: per (tile, window, matrix) one lane block of fp4 codes and its scale against the
// window's fp8 hi and lo operands: two scaled matrix-core instructions
template <int WPW>
__device__ __forceinline__ void gu_math_mx(f32x4 (&acc)[GU_MX_RT][2], const GUItem<WPW>& T, const XMX<WPW>& xm) {
#pragma unroll
  for (int tl = 0; tl < GU_MX_RT; ++tl) acc[tl][0] = acc[tl][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int tl = 0; tl < GU_MX_RT; ++tl)
#pragma unroll
    for (int wi = 0; wi < WPW; ++wi)
#pragma unroll
      for (int mat = 0; mat < 2; ++mat) {
        const u32x4 c = T.v[(tl * WPW + wi) * 2 + mat];
        const uint32_t sa = T.sc[(tl * WPW + wi) * 2 + mat];
        acc[tl][mat] = mfma_mx(c, sa, xm.hi[wi][0], xm.hi[wi][1], xm.sc[wi], 0, acc[tl][mat]);
        acc[tl][mat] = mfma_mx(c, sa, xm.lo[wi][0], xm.lo[wi][1], xm.sc[wi], 1, acc[tl][mat]);
      }
}

template <int WPW>
__device__ __forceinline__ void gu_load_xb(u32x4 (&xb)[WPW][4][2], const u32x4* xf, int win0, bool active,
                                           int lane) {
#pragma unroll
  for (int wi = 0; wi < WPW; ++wi)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl)
        xb[wi][j][hl] = active ? ld16(xf + ((size_t)((win0 + wi) * 4 + j) * 2 + hl) * 64 + lane)
                               : u32x4{0u, 0u, 0u, 0u};
}

// Item schedule of the gate/up and down kernels (routed items; the shared expert's items go to
// workgroups b < n_sh first).
//  * Static part: rounds 0 .. S-1; in round s workgroup b takes item s G + f with
//    f = (b - n_sh) mod G, i.e. the workgroups that took a shared item start the routed deal last.
//    With at least 6 rounds of items S = n / G - 2 and the rest is claimed; with fewer, every
//    round is static.
//  * Claimed part: items S G .. n-1, split into P = min(NGRP, G / 8) interleaved pools (item
//    S G + p + P c for pool p and counter value c). Workgroup b draws from pool (b / 8) mod P, so
//    every pool has members (workgroup 8 p is one) and is served by workgroups on all XCDs
//    (consecutive workgroups go to different XCDs): the XCDs of this part stream at noticeably different rates,
//    which a fully static deal turns into a tail, and claiming lets the faster ones take more.
//    Device-scope atomics on one address serialise (about 30 ns each), hence several pools, and
//    only the last rounds are claimed.
//  * Vector memory results complete in issue order, so a claim is issued right after an item's
//    loads and its result is stored (into the LDS ring that the epilogues publish) two items
//    later; it never holds up a load that is needed sooner.
constexpr int NGRP = 8;          // claim pools
constexpr int CTR_STRIDE = 64;   // uint32 words between pool counters (256 B)
// Counters of the one-launch layer kernel, zeroed by the router, each NPC slots 256 B apart:
// completed gate/up items, then completed down items. Workgroup b adds to slot b mod NPC: adds to
// one address serialise (about 30 ns each), and 256 workgroups counting into a single word took
// about 8 us.
constexpr int NPC = 16;
constexpr int CT_GU = 2 * NGRP;
constexpr int CT_DN = CT_GU + NPC;
constexpr int N_CTR = CT_DN + NPC;
struct Sched {
  int G, S, f, pool, npool;  // workgroups, static rounds, first item, pool, pools
  bool claims;               // whether the last rounds are claimed
  uint32_t* ctr;             // this workgroup's pool counter
};
// With ipe_xcd > 0 (the down kernel: ipe_xcd items per expert), a static round deals whole
// experts round-robin over the XCDs (consecutive workgroup ids go to different XCDs): expert
// block i of the round goes to XCD i mod 8, and its items to consecutive workgroups there. Every
// item of an expert reads the expert's activation fragments, which are then fetched into one
// XCD's L2 instead of all eight, and a round with few experts still spans every XCD. Within each
// XCD the shared-item workgroups start the deal last. Needs G/8 to be a multiple of ipe_xcd.
__device__ __forceinline__ Sched make_sched(int n, int G, int b, int n_sh, uint32_t* ctr_base,
                                            int ipe_xcd = 0) {
  Sched q;
  q.G = G;
  q.claims = n >= 6 * G;
  q.S = q.claims ? n / G - 2 : (n + G - 1) / G;
  const int g8 = G >> 3;
  if (ipe_xcd > 0 && G % 8 == 0 && g8 % ipe_xcd == 0) {
    const int j = ((b >> 3) - (n_sh + 7) / 8 + g8) % g8;  // slot within the XCD
    q.f = (((j / ipe_xcd) << 3) + (b & 7)) * ipe_xcd + j % ipe_xcd;
  } else {
    q.f = (b - n_sh + G) % G;
  }
  q.npool = min(NGRP, max(1, G >> 3));
  q.pool = (b >> 3) % q.npool;
  q.ctr = ctr_base + q.pool * CTR_STRIDE;
  return q;
}
__device__ __forceinline__ bool is_static(const Sched& q, int h) { return !q.claims || h < q.S; }
// item of step h if it is static (h < S)
__device__ __forceinline__ int static_item(const Sched& q, int h) { return h * q.G + q.f; }
// item for counter value c of this workgroup's pool
__device__ __forceinline__ int pool_item(const Sched& q, uint32_t c) { return q.S * q.G + q.pool + q.npool * (int)c; }
__device__ __forceinline__ uint32_t claim_raw(uint32_t* ctr) {
  return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The woken-expert list held across the lanes of every wave: lane l keeps entries l, l + 64, ...
// A lookup is v_readlane with a uniform lane index, so an item descriptor is computed without
// writing any VGPR: the streaming loops then never overwrite, between an epilogue's stores and
// the next loads, a register that the waitcnt logic would have to drain first.
struct Woken {
  int v[MAX_U / 64];
};
__device__ __forceinline__ Woken load_woken(const Smem& S, int lane) {
  Woken w;
#pragma unroll
  for (int m = 0; m < MAX_U / 64; ++m) w.v[m] = S.woken[lane + 64 * m];
  return w;
}
__device__ __forceinline__ uint32_t woken_at(const Woken& w, int u) {  // u wave-uniform
  const int l = u & 63, m = u >> 6;
  int e = __builtin_amdgcn_readlane(w.v[0], l);
#pragma unroll
  for (int i = 1; i < MAX_U / 64; ++i)
    if (m == i) e = __builtin_amdgcn_readlane(w.v[i], l);
  return (uint32_t)e;
}

// Routed item `idx` (or a valid stand-in when idx is out of range, so that every path issues
// the same loads).
template <bool MX>
__device__ __forceinline__ GUDesc gu_desc(const Args& a, const Woken& wk, int idx, int n_items, int ipe) {
  const int it = (idx >= 0 && idx < n_items) ? idx : 0;
  GUDesc d;
  d.u = it / ipe;
  d.ntile = MX ? GU_MX_RT : 1;
  d.row0 = (it % ipe) * 16 * d.ntile;
  const uint32_t e = woken_at(wk, d.u);
  const uint32_t row = e * (uint32_t)a.I + (uint32_t)d.row0;  // tensor row of the item's first tile
  if (MX) {
    d.off = row * (uint32_t)(a.H / 2);
    d.soff = row * (uint32_t)(a.H / 32);
  } else {
    d.off = row * (uint32_t)(a.H * 2);
    d.soff = 0;
  }
  return d;
}

template <int WPW, bool MX>
__device__ __forceinline__ void gu_load(GUItem<WPW>& T, const GURes& R, const GUDesc& d, int H, uint32_t vbc,
                                        uint32_t vbs) {
  if (MX) gu_load_mx<WPW>(T, R, d, H, vbc, vbs);
  else gu_load_bf16<WPW>(T, R.g, R.u, d.off, vbc);
}

template <int WPW, bool MX>
__device__ __forceinline__ void gu_math(f32x4 (&acc)[GU_MX_RT][2], const GUItem<WPW>& T,
                                        const u32x4 (&xb)[WPW][4][2], const XMX<WPW>& xm) {
  if constexpr (MX) gu_math_mx<WPW>(acc, T, xm);
  else gu_math_bf16<WPW>(acc, T, xb);
}

// ------------------------------------------------------------------------------------------
// down items. NWIN = I / 128 windows; wave w owns window w % NWIN and tile group
// w / NWIN, with TPW row tiles. An mxfp4 item has as many rows as a bf16 one (a quarter of its
// bytes): with 256-row mxfp4 items a k = 16 layer had about 3.2 items per workgroup, too few for
// the claimed rounds, and its partial last round cost more than the smaller items' extra epilogues.
// ------------------------------------------------------------------------------------------
template <int NWIN>
struct DnShape {
  static constexpr int WPWIN = NW / NWIN;                   // waves per window
  static constexpr int TPI_BF = NWIN == 8 ? 4 : 8;           // row tiles per bf16 item
  static constexpr int TPW_BF = TPI_BF / WPWIN;              // row tiles per wave, bf16
  static constexpr int TPI_MX = TPI_BF;                      // row tiles per mxfp4 item
  static constexpr int TPW_MX = TPW_BF;
};

template <int NWIN>
struct DNItem {
  u32x4 v[DnShape<NWIN>::TPW_BF * 4];  // bf16: [tile*4 + j]; mxfp4: [tile] (first TPW_MX entries)
  uint32_t sc[DnShape<NWIN>::TPW_MX];
};

struct DNDesc {
  int u, row0, ntile;
  uint32_t off;   // byte offset of the item in the down tensor (codes for mxfp4)
  uint32_t soff;  // byte offset of the item's scales (mxfp4)
};

template <int NWIN, bool MX>
__device__ __forceinline__ DNDesc dn_desc(const Args& a, const Woken& wk, int idx, int n_items, int ipe) {
  using SH = DnShape<NWIN>;
  const int it = (idx >= 0 && idx < n_items) ? idx : 0;
  DNDesc d;
  d.u = it / ipe;
  d.ntile = MX ? SH::TPI_MX : SH::TPI_BF;
  d.row0 = (it % ipe) * 16 * d.ntile;
  const uint32_t e = woken_at(wk, d.u);
  const uint32_t row = e * (uint32_t)a.H + (uint32_t)d.row0;  // tensor row of the item's first tile
  if (MX) {
    d.off = row * (uint32_t)(a.I / 2);
    d.soff = row * (uint32_t)(a.I / 32);
  } else {
    d.off = row * (uint32_t)(a.I * 2);
    d.soff = 0;
  }
  return d;
}

// bf16 item (tiled layout): wave (window win, tile group tg) reads, for each of its tiles, the
// window's four 1 KiB fragment tiles (4 KiB contiguous).
template <int NWIN>
__device__ __forceinline__ void dn_load_bf16(DNItem<NWIN>& T, rsrc_t rw, uint32_t soff, int I, int wave, int lane) {
  using SH = DnShape<NWIN>;
  const int win = wave % NWIN, tg = wave / NWIN;
  const uint32_t vb = (uint32_t)(256 * win + lane) * 16u;
#pragma unroll
  for (int tl = 0; tl < SH::TPW_BF; ++tl) {
    const uint32_t st = soff + (uint32_t)((tg * SH::TPW_BF + tl) * 16 * I * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) T.v[tl * 4 + j] = bld16(rw, vb + j * 1024, st);
  }
}

// mxfp4 item (tiled layout): per (tile, window) 1 KiB of codes and 64 B of scales
template <int NWIN>
__device__ __forceinline__ void dn_load_mx(DNItem<NWIN>& T, rsrc_t rw, rsrc_t rs, const DNDesc& d, int I, int wave,
                                           int lane) {
  using SH = DnShape<NWIN>;
  const int win = wave % NWIN, tg = wave / NWIN;
#pragma unroll
  for (int tl = 0; tl < SH::TPW_MX; ++tl) {
    const int tile = tg * SH::TPW_MX + tl;
    T.v[tl] = bld16(rw, (uint32_t)(win * 64 + lane) * 16u, d.off + (uint32_t)(tile * 16 * (I / 2)));
    T.sc[tl] = bld1(rs, (uint32_t)(win * 64 + lane), d.soff + (uint32_t)(tile * 16 * (I / 32)));
  }
}

template <int NWIN, bool MX>
__device__ __forceinline__ void dn_load(DNItem<NWIN>& T, rsrc_t rw, rsrc_t rs, const DNDesc& d, int I, int wave,
                                        int lane) {
  if (MX) dn_load_mx<NWIN>(T, rw, rs, d, I, wave, lane);
  else dn_load_bf16<NWIN>(T, rw, d.off, I, wave, lane);
}

// B fragments (down activations) of this wave's window for one expert slot
template <int NWIN>
__device__ __forceinline__ void dn_load_b(u32x4 (&bf)[4][2], rsrc_t raf, uint32_t soff, int wave, int lane) {
  const int win = wave % NWIN;
  const uint32_t vb = (uint32_t)(512 * win + lane) * 16u;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) bf[j][hl] = bld16_cached(raf, vb + (uint32_t)((j * 2 + hl) * 1024), soff);
}

// B operands of a wave's window for one expert slot: bf16 hi/lo fragments (4 k-steps), or the
// MX-fp8 hi/lo operands and their scale word (mxfp4 routed experts)
struct DBF {
  u32x4 f[4][2];
};
struct DBM {
  u32x4 hi[2], lo[2];
  uint32_t sc;
};
template <bool MX>
using DnB = std::conditional_t<MX, DBM, DBF>;

template <int NWIN, bool MX>
__device__ __forceinline__ void dn_load_bb(DnB<MX>& B, rsrc_t raf, int u, int I, int wave, int lane) {
  if constexpr (MX) {
    const uint32_t soff = (uint32_t)((u * (I / WIN) + wave % NWIN) * MXW);
    const uint32_t vb = (uint32_t)lane * 32u;
    B.hi[0] = bld16_cached(raf, vb, soff);
    B.hi[1] = bld16_cached(raf, vb + 16u, soff);
    B.lo[0] = bld16_cached(raf, vb + 2048u, soff);
    B.lo[1] = bld16_cached(raf, vb + 2064u, soff);
    B.sc = __builtin_amdgcn_raw_buffer_load_b32(raf, (uint32_t)(4096 + lane * 4), soff, 0);
  } else {
    dn_load_b<NWIN>(B.f, raf, (uint32_t)(u * (I / 32) * 2048), wave, lane);
  }
}

template <int NWIN, bool MX>
__device__ __forceinline__ void dn_math(f32x4 (&acc)[DnShape<NWIN>::TPW_MX], const DNItem<NWIN>& T,
                                        const DnB<MX>& B) {
  using SH = DnShape<NWIN>;
#pragma unroll
  for (int tl = 0; tl < SH::TPW_MX; ++tl) acc[tl] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (MX) {  // per tile: the lane's fp4 block and scale against the fp8 hi and lo operands
#pragma unroll
    for (int tl = 0; tl < SH::TPW_MX; ++tl) {
      acc[tl] = mfma_mx(T.v[tl], T.sc[tl], B.hi[0], B.hi[1], B.sc, 0, acc[tl]);
      acc[tl] = mfma_mx(T.v[tl], T.sc[tl], B.lo[0], B.lo[1], B.sc, 1, acc[tl]);
    }
  } else {
#pragma unroll
    for (int tl = 0; tl < SH::TPW_BF; ++tl)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[tl] = mfma16(T.v[tl * 4 + j], B.f[j][0], acc[tl]);
        acc[tl] = mfma16(T.v[tl * 4 + j], B.f[j][1], acc[tl]);
      }
  }
}

template <int NWIN>
__device__ __forceinline__ void dn_store_partial(Smem& S, const f32x4* acc, int tpw, int wave, int lane) {
  const int win = wave % NWIN, tg = wave / NWIN;
  for (int tl = 0; tl < tpw; ++tl)
    *reinterpret_cast<f32x4*>(&S.red[((win + NWIN * tg) * tpw + tl) * 256 + lane * 4]) = acc[tl];
}

// Reduce the item's partial tiles over windows and write the P rows of the tokens routed to it.
template <int NWIN>
__device__ void dn_epilogue(const Args& a, Smem& S, int ntile, int tpw, int u, bool routed, int row0,
                            int tid, int ring = -1, int* next = nullptr) {
  const int H = a.H, K = a.K, k = a.k;
  __syncthreads();
  if (ring >= 0) {  // the next item index, read before this epilogue's stores are issued
    *next = __builtin_amdgcn_readfirstlane(S.claim[ring]);
    __builtin_amdgcn_sched_barrier(0);
  }
  {
    const int r = tid & 15, c = (tid >> 4) & 15, par = tid >> 8;  // par: tile parity
    int slot = -1;
    if (c < k) slot = routed ? (int)S.slot[u][c] : K;
    if (slot >= 0) {
      float* dst = a.part + ((size_t)c * (K + 1) + slot) * H + row0 + r;
      const int idx = (c + 16 * (r >> 2)) * 4 + (r & 3);
      for (int tl = par; tl < ntile; tl += 2) {
        const int tg = tl / tpw, lt = tl % tpw;  // tile tl: tile group tg, local tile lt
        float v = 0.f;
#pragma unroll
        for (int win = 0; win < NWIN; ++win) v += S.red[((win + NWIN * tg) * tpw + lt) * 256 + idx];
        st_dev(dst + tl * 16, v);  // published inside the launch
      }
    }
  }
  __syncthreads();  // the next item's partial tiles reuse S.red
}

// y[t][h] = sum_j P[t][j][h] + P[t][K][h] (+ x[t][h]). Four threads per four outputs: thread g
// of the quad sums terms g, g + 4, ... (the routed slots, then the shared expert's, then the
// residual), each term one float4 load, all issued before any is added; a quad reduction by DPP,
// (s0 + s1) + (s2 + s3), finishes the sum, in the same order on every run. One thread with every
// term in a loop waited for each load in turn.
constexpr int CMB_T = 5;  // terms per thread: at most 16 routed + shared + residual = 18 <= 4 x 5
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));  // [1,0,3,2]
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));  // [2,3,0,1]
}
// Output float4 o of y, thread g of its quad (every lane takes part in the DPP steps; live: o is an
// output). The partial rows were published inside the same launch and are read past the L2.
__device__ __forceinline__ void combine_quad(const Args& a, int o, int g, bool live) {
  const int H = a.H, K = a.K, H4 = H / 4;
  const int oc = live ? o : 0, t = oc / H4, c = oc % H4;
  const int nr = K + (a.Is > 0 ? 1 : 0);   // partial rows of the token
  const int n = nr + (a.residual ? 1 : 0);  // terms
  const float4* p = reinterpret_cast<const float4*>(a.part + (size_t)t * (K + 1) * H) + c;
  const float4* xr = reinterpret_cast<const float4*>(a.x + (size_t)t * H) + c;
  const rsrc_t rp = buf_rsrc(a.part, (uint32_t)((size_t)a.k * (K + 1) * H * 4));
  float4 v[CMB_T];
#pragma unroll
  for (int i = 0; i < CMB_T; ++i) {
    const int j = g + 4 * i, jj = j < n ? j : 0;  // terms past n re-read term 0 and are unused
    if (jj < nr) {
      const uint32_t off = (uint32_t)((((size_t)t * (K + 1) + jj) * H + 4 * c) * 4);
      v[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, BUF_DEV));
    } else {
      v[i] = *xr;
    }
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < CMB_T; ++i)
    if (g + 4 * i < n) { acc.x += v[i].x; acc.y += v[i].y; acc.z += v[i].z; acc.w += v[i].w; }
  acc.x = quad_sum(acc.x); acc.y = quad_sum(acc.y); acc.z = quad_sum(acc.z); acc.w = quad_sum(acc.w);
  if (live && g == 0) reinterpret_cast<float4*>(a.y + (size_t)t * H)[c] = acc;
}

// ------------------------------------------------------------------------------------------
// phase counters of the one-launch layer kernel
// ------------------------------------------------------------------------------------------
// Publishing inside the one-launch layer kernel: the data is written with device-coherent stores,
// so it is visible everywhere once the stores are complete (s_waitcnt); no L2 write-back is needed
// before the count that announces it.
//
// Adds this workgroup's item count to a phase counter once every wave's stores are complete.
__device__ __forceinline__ void publish_count(const Args& a, int ct, int n, int tid) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores (and loads) are complete
  __syncthreads();                // and every other wave's
  if (tid == 0 && n > 0)
    __hip_atomic_fetch_add(a.ctr + (ct + (int)(blockIdx.x % NPC)) * CTR_STRIDE, (uint32_t)n, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

constexpr uint32_t WAIT_POLLS = 1u << 22;
// Waits until a phase counter's slots sum to `target`: lane i < NPC of wave 0 reads slot i per
// poll (one round trip), and the workgroup meets at a barrier. Bounded: after WAIT_POLLS polls
// (seconds) the call is reported failed (n_woken = -1) and the workgroup goes on, so no wave ever
// hangs.
__device__ __forceinline__ void wait_count(const Args& a, int ct, uint32_t target, int tid) {
  if (tid < 64) {
    uint32_t* slot = a.ctr + (ct + (tid < NPC ? tid : 0)) * CTR_STRIDE;
    for (uint32_t polls = 0;; ++polls) {
      uint32_t v = tid < NPC ? __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
#pragma unroll
      for (int off = NPC / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);  // lanes 0 .. NPC-1 hold the sum
      if (__builtin_amdgcn_readfirstlane(v) >= target) break;
      if (polls == WAIT_POLLS) {
        if (tid == 0 && a.out_n) st_dev(reinterpret_cast<uint32_t*>(a.out_n), 0xFFFFFFFFu);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------------------------------
// kernels
// ------------------------------------------------------------------------------------------
template <bool MX>
__global__ void __launch_bounds__(NTH) k_router(Args a) {
  __shared__ RouterSmem S;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  // this layer's claim pools and the counters of the one-launch layer kernel start at 0
  for (int i = blockIdx.x * NTH + tid; i < N_CTR; i += gridDim.x * NTH) a.ctr[i * CTR_STRIDE] = 0u;
  router_item<MX>(a, S, blockIdx.x, wave, lane, tid);
}

// The gate/up work of one workgroup: the routing prologue (into LDS), the shared expert's row tile
// when b < Is/16, then its routed items. Returns the number of items it completed. The activation
// fragments are published inside the launch (device-coherent stores).
template <int WPW, bool MX>
__device__ __forceinline__ int gateup_body(const Args& a, Smem& S, int tid, int lane, int wave) {
  const int H = a.H, I = a.I, Is = a.Is;
  const int G = gridDim.x, b = blockIdx.x;
  const int win0 = wave * WPW;
  const bool active = win0 < H / WIN;  // H is a multiple of 128 * WPW
  const int wsafe = active ? win0 : 0; // inactive waves load window 0 and multiply it by zero

  // Item sequence: the shared expert's row tiles (known before routing, so their weights are
  // requested first), then the routed items (see make_sched).
  const int n_sh = Is / 16;
  GUItem<WPW> Ts;
  const uint32_t E = a.E;
  GURes R;
  const uint32_t wbytes = MX ? E * I * (H / 2) : E * I * H * 2;
  R.g = buf_rsrc(a.wg, wbytes);
  R.u = buf_rsrc(a.wu, wbytes);
  R.sg = buf_rsrc(a.sg, MX ? E * I * (H / 32) : 0);
  R.su = buf_rsrc(a.su, MX ? E * I * (H / 32) : 0);
  const uint32_t vbb = (uint32_t)(256 * wsafe + lane) * 16u;            // bf16 tiles
  const uint32_t vbc = MX ? (uint32_t)(64 * wsafe + lane) * 16u : vbb;  // this layer's tiles
  const uint32_t vbs = (uint32_t)(64 * wsafe + lane);                   // mxfp4 scales
  const RoutePart rp = route_issue(a, tid);
  __builtin_amdgcn_sched_barrier(0);  // the partials are requested ahead of the shared tile
  {  // every workgroup issues the tile's loads (the same count of loads in flight on every path,
     // so waiting for the partials never waits for the tile); without a shared item the resource
     // is empty and the loads return zeros without a memory access
    const uint32_t shb = b < n_sh ? (uint32_t)(Is * H * 2) : 0u;
    gu_load_bf16<WPW>(Ts, buf_rsrc(a.shg, shb), buf_rsrc(a.shu, shb), b < n_sh ? (uint32_t)(b * 16 * H * 2) : 0u, vbb);
  }
  route(a, S, rp, wave, lane, tid);
  const int U = __builtin_amdgcn_readfirstlane(S.nw);

  // B operands of this wave's H windows (the raw block), used by every item: bf16 hi/lo
  // fragments (bf16 layers and the shared expert's bf16 tiles), MX-fp8 hi/lo operands (mxfp4
  // routed experts)
  u32x4 xb[WPW][4][2];
  XMX<WPW> xm;
  if (!MX || b < n_sh) gu_load_xb<WPW>(xb, MX ? a.xfrag_sh : a.xfrag, win0, active, lane);
  if (MX && b >= n_sh) gu_load_xmx<WPW>(xm, a.xfrag, win0, active, lane);

  const int ipe = I / (16 * (MX ? GU_MX_RT : 1));
  const int n_gu = U * ipe;
  int n_done = 0;
  if (b < n_sh) {
    f32x4 acc[GU_MX_RT][2];
    gu_math_bf16<WPW>(acc, Ts, xb);
    gu_epilogue<false>(a, S, acc, 1, U, b * 16, false, wave, lane, tid);
    if (MX) gu_load_xmx<WPW>(xm, a.xfrag, win0, active, lane);
    n_done = 1;
  }

  // Routed items (see make_sched), D items deep: at step h item h is multiplied while the loads
  // of items h + 1 .. h + D - 1 are in flight (those of item h + D - 1 issued at the top of the
  // step). Thread 0 stores the index of item h + D into the LDS ring (static, or claimed two steps
  // earlier) and claims item h + D + 2 when that one is claimed; the epilogue reads item h + D back
  // for the next step's loads. Claims whose step would be negative are taken before the loop.
  // Two in flight: for mxfp4 items (70 KB) four were measured slower (more stand-in loads when a
  // workgroup has few items, and no gain in the steady state).
  constexpr int D = 2;
  const Sched q = make_sched(n_gu, G, b, n_sh, a.ctr);
  const int r0 = static_item(q, 0);
  if (r0 >= n_gu) return n_done;  // every later item is past the end too
  const Woken wk = load_woken(S, lane);
  GUItem<WPW> T[D];
  GUDesc dd[D];
  int nx[D];
#pragma unroll
  for (int j = 0; j + 1 < D; ++j) {
    nx[j] = static_item(q, j);
    dd[j] = gu_desc<MX>(a, wk, nx[j], n_gu, ipe);  // a valid stand-in past the end
    gu_load<WPW, MX>(T[j], R, dd[j], H, vbc, vbs);
  }
  int nload = static_item(q, D - 1);  // item of the next step whose loads are issued
  // Claims (thread 0): the claim for item X sits in cl[X & 1]. It is issued behind the loads of
  // step X - D - 1 (item X - 2 with two in flight), so it returns right after them, and it is read
  // after the math of step X - D, which waits for those loads anyway: a workgroup holds at most one
  // claimed item that it has not started loading, which keeps the end spread to about one item.
  static_assert(D == 2, "the claim timing assumes two items in flight");
  uint32_t cl[2] = {0u, 0u};
  if (tid == 0 && !is_static(q, D)) cl[D & 1] = claim_raw(q.ctr);
  for (int h = 0;; h += D) {
    bool done = false;
#pragma unroll
    for (int r = 0; r < D; ++r) {
      const int st = h + r;
      const int jl = (r + D - 1) % D;  // buffer of item st + D - 1
      nx[jl] = nload;
      dd[jl] = gu_desc<MX>(a, wk, nload, n_gu, ipe);
      gu_load<WPW, MX>(T[jl], R, dd[jl], H, vbc, vbs);
      if (tid == 0 && !is_static(q, st + D + 1)) cl[(st + D + 1) & 1] = claim_raw(q.ctr);
      __builtin_amdgcn_sched_barrier(0);
      {
        f32x4 acc[GU_MX_RT][2];
        gu_math<WPW, MX>(acc, T[r], xb, xm);
        if (tid == 0)  // item st + D, read back by this step's epilogue after its barriers
          S.claim[(st + D) & 3] = is_static(q, st + D) ? static_item(q, st + D) : pool_item(q, cl[(st + D) & 1]);
        gu_epilogue<MX>(a, S, acc, dd[r].ntile, dd[r].u, dd[r].row0, true, wave, lane, tid, (st + D) & 3, &nload);
      }
      ++n_done;  // every step's item is inside the list (the loop stops before a step past the end)
      if (nx[(r + 1) % D] >= n_gu) { done = true; break; }  // the next step's item is past the end
    }
    if (done) break;
  }
  return n_done;
}

// The down work of one workgroup, after its gate/up items: the shared expert's row group when
// b < n_sh, then its routed items. The routing tables are in LDS (the routing prologue of the same
// launch); the activation fragments were published inside the launch, and the partial rows are
// published the same way. Returns the number of items it completed.
template <int NWIN, bool MX>
__device__ __forceinline__ int down_body(const Args& a, Smem& S, int tid, int lane, int wave) {
  using SH = DnShape<NWIN>;
  constexpr int TPW = MX ? SH::TPW_MX : SH::TPW_BF;
  const int H = a.H, I = a.I, Is = a.Is;
  const int G = gridDim.x, b = blockIdx.x;

  // Item sequence: the shared expert's row groups (requested first), then the routed items
  // (see make_sched).
  const int n_sh = Is > 0 ? H / (16 * SH::TPI_BF) : 0;
  DNItem<NWIN> Ts;
  const uint32_t E = a.E;
  const rsrc_t rw = buf_rsrc(a.wd, MX ? E * H * (I / 2) : E * H * I * 2);
  const rsrc_t rs = buf_rsrc(a.sd, MX ? E * H * (I / 32) : 0);
  const rsrc_t raf = buf_rsrc(a.afrag, MX ? (uint32_t)a.umax * (I / WIN) * MXW : (uint32_t)a.umax * (I / 32) * 2048);
  if (b < n_sh) dn_load_bf16<NWIN>(Ts, buf_rsrc(a.shd, H * Is * 2), (uint32_t)(b * 16 * SH::TPI_BF * Is * 2), Is, wave, lane);

  const int U = __builtin_amdgcn_readfirstlane(S.nw);

  const int ipe = H / (16 * (MX ? SH::TPI_MX : SH::TPI_BF));
  const int n_dn = U * ipe;
  constexpr int D = 2;
  const Sched q = make_sched(n_dn, G, b, n_sh, a.ctr + NGRP * CTR_STRIDE, ipe);
  const int q0 = static_item(q, 0);
  const Woken wk = load_woken(S, lane);
  DNItem<NWIN> T[D];
  DnB<MX> Bf[D];
  DNDesc dd[D];
  int nx[D];
  // The first routed items' weights are requested before the wait for the activations (they do
  // not depend on them), so the stream goes on while the last gate/up items finish elsewhere:
  // one item (bf16, 128 KB), or both buffers' items (mxfp4, 34 KB each); two bf16 items would
  // not fit the registers next to a shared item.
  constexpr int NPRE = MX ? D : D - 1;
  if (q0 < n_dn) {
#pragma unroll
    for (int j = 0; j < NPRE; ++j) {
      nx[j] = static_item(q, j);
      dd[j] = dn_desc<NWIN, MX>(a, wk, nx[j], n_dn, ipe);  // a valid stand-in past the end
      dn_load<NWIN, MX>(T[j], rw, rs, dd[j], I, wave, lane);
    }
  }
  {  // every gate/up item of the launch (routed and shared) is complete
    const uint32_t gu_total = (uint32_t)(U * (I / (16 * (MX ? GU_MX_RT : 1))) + Is / 16);
    wait_count(a, CT_GU, gu_total, tid);
  }

  int n_done = 0;
  if (b < n_sh) {
    DBF bs;
    dn_load_b<NWIN>(bs.f, buf_rsrc(a.afrag_sh, (Is / 32) * 2048), 0u, wave, lane);
    f32x4 acc[SH::TPW_MX];
    dn_math<NWIN, false>(acc, Ts, bs);
    dn_store_partial<NWIN>(S, acc, SH::TPW_BF, wave, lane);
    dn_epilogue<NWIN>(a, S, SH::TPI_BF, SH::TPW_BF, U, false, b * 16 * SH::TPI_BF, tid);
    n_done = 1;
  }
  // Routed items, scheduled and pipelined as in the gate/up kernel (D items deep: at step h item
  // h is multiplied while the weights and activation fragments of items h + 1 .. h + D - 1 are in
  // flight). Two in flight for both formats: with the 34 KB mxfp4 items, three or four in flight
  // were measured slower (k = 16: 22.6 and 22.0 us against 19.9).
  if (q0 >= n_dn) return n_done;  // every later item is past the end too
#pragma unroll
  for (int j = 0; j < NPRE; ++j) dn_load_bb<NWIN, MX>(Bf[j], raf, dd[j].u, I, wave, lane);
  int nload = static_item(q, D - 1);  // item of the next step whose loads are issued
  // Claims (thread 0): the claim for item X sits in cl[X & 1]. It is issued behind the loads of
  // step X - D - 1 (item X - 2 with two in flight), so it returns right after them, and it is read
  // after the math of step X - D, which waits for those loads anyway: a workgroup holds at most one
  // claimed item that it has not started loading, which keeps the end spread to about one item.
  static_assert(D == 2, "the claim timing assumes two items in flight");
  uint32_t cl[2] = {0u, 0u};
  if (tid == 0 && !is_static(q, D)) cl[D & 1] = claim_raw(q.ctr);
  // Step st: request item st + D - 1 (unless already requested), multiply item st, publish it.
  // Returns whether the next step's item is past the end.
  auto step = [&](const int st, const int r, const bool load) __attribute__((always_inline)) {
    const int jl = (r + D - 1) % D;  // buffer of item st + D - 1
    if (load) {
      nx[jl] = nload;
      dd[jl] = dn_desc<NWIN, MX>(a, wk, nload, n_dn, ipe);
      dn_load<NWIN, MX>(T[jl], rw, rs, dd[jl], I, wave, lane);
      dn_load_bb<NWIN, MX>(Bf[jl], raf, dd[jl].u, I, wave, lane);
    }
    if (tid == 0 && !is_static(q, st + D + 1)) cl[(st + D + 1) & 1] = claim_raw(q.ctr);
    __builtin_amdgcn_sched_barrier(0);
    {
      f32x4 acc[SH::TPW_MX];
      dn_math<NWIN, MX>(acc, T[r], Bf[r]);
      if (tid == 0)  // item st + D, read back by this step's epilogue after its barrier
        S.claim[(st + D) & 3] = is_static(q, st + D) ? static_item(q, st + D) : pool_item(q, cl[(st + D) & 1]);
      dn_store_partial<NWIN>(S, acc, TPW, wave, lane);
      dn_epilogue<NWIN>(a, S, dd[r].ntile, TPW, dd[r].u, true, dd[r].row0, tid, (st + D) & 3, &nload);
    }
    ++n_done;
    return nx[(r + 1) % D] >= n_dn;
  };
  // The first round is peeled off: with NPRE == D its first step requests nothing. A step whose
  // loads depend on the iteration made the compiler wait for every load in flight (the next
  // item's too) before that step's products, once per round.
  bool done = false;
#pragma unroll
  for (int r = 0; r < D && !done; ++r) done = step(r, r, NPRE < D || r > 0);
  for (int h = D; !done; h += D) {
#pragma unroll
    for (int r = 0; r < D && !done; ++r) done = step(h + r, r, true);
  }
  return n_done;
}

// One MoE layer's expert work in one launch: the routing prologue and the gate/up items, then the
// down items, then the combine, each phase starting when the previous one is complete on every
// workgroup. A phase publishes its results with device-coherent stores; each workgroup, once its
// stores are complete, adds its item count to the phase's counter (zeroed by the router kernel),
// and the next phase waits for the counter to reach the phase's item total. So no kernel
// boundary sits between the phases: a workgroup that finishes its gate/up items early already
// streams its first down items' weights while the last gate/up items finish elsewhere, and the
// down phase finds the routing tables in LDS. The waits cannot deadlock: a phase's items never
// wait on anything, and every workgroup runs its items of a phase before it waits for the next;
// a wait that runs past its bound reports the call as failed.
template <int WPW, int NWIN, bool MX>
__global__ void __launch_bounds__(NTH) k_layer(Args a) {
  using SH = DnShape<NWIN>;
  __shared__ Smem S;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int H = a.H, Is = a.Is;
  const int n_gu = gateup_body<WPW, MX>(a, S, tid, lane, wave);
  publish_count(a, CT_GU, n_gu, tid);
  const int n_dn = down_body<NWIN, MX>(a, S, tid, lane, wave);
  publish_count(a, CT_DN, n_dn, tid);
  // the combine: workgroup b < ceil(k H / 512) takes 128 output float4s, four threads each
  const int n_out = a.k * (H / 4);
  if ((int)blockIdx.x * 128 < n_out) {
    const uint32_t U = (uint32_t)__builtin_amdgcn_readfirstlane(S.nw);
    const uint32_t dn_total = U * (uint32_t)(H / (16 * (MX ? SH::TPI_MX : SH::TPI_BF))) +
                              (Is > 0 ? (uint32_t)(H / (16 * SH::TPI_BF)) : 0u);
    wait_count(a, CT_DN, dn_total, tid);
    const int o = (int)blockIdx.x * 128 + (tid >> 2);
    combine_quad(a, o, tid & 3, o < n_out);
  }
}

// ------------------------------------------------------------------------------------------
// weight packing: row-major expert matrices -> fragment tiles (a pure permutation)
// ------------------------------------------------------------------------------------------
// bf16: 16-byte chunk c of the tiled array is (matrix m, row tile rt, k-step s, lane l) and holds
// row 16 rt + l % 16, columns 32 s + 8 (l / 16) .. +7.
__global__ void __launch_bounds__(256) k_pack_bf16(const uint8_t* src, uint8_t* dst, int rows, int cols,
                                                   uint64_t n_chunks) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  const uint64_t per_mat = (uint64_t)rows * cols / 8;
  const int ks = cols / 32;
  for (uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n_chunks; c += stride) {
    const uint64_t m = c / per_mat, rem = c % per_mat;
    const int l = (int)(rem % 64), s = (int)((rem / 64) % ks), rt = (int)(rem / 64 / ks);
    const uint64_t from = m * per_mat * 16 + ((uint64_t)(16 * rt + (l & 15)) * cols + 32 * s + 8 * (l >> 4)) * 2;
    *reinterpret_cast<u32x4*>(dst + c * 16) = *reinterpret_cast<const u32x4*>(src + from);
  }
}

// mxfp4: codes chunk c is (matrix m, row tile rt, window w, lane l) = the 16 code bytes of block
// 4 w + l / 16 of row 16 rt + l % 16; scale byte c is that block's scale.
__global__ void __launch_bounds__(256) k_pack_mx(const uint8_t* src, const uint8_t* src_s, uint8_t* dst,
                                                 uint8_t* dst_s, int rows, int cols, uint64_t n_blocks) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  const uint64_t per_mat = (uint64_t)rows * cols / 32;
  const int nw = cols / 128;
  for (uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n_blocks; c += stride) {
    const uint64_t m = c / per_mat, rem = c % per_mat;
    const int l = (int)(rem % 64), w = (int)((rem / 64) % nw), rt = (int)(rem / 64 / nw);
    const uint64_t blk = m * per_mat + (uint64_t)(16 * rt + (l & 15)) * (cols / 32) + 4 * w + (l >> 4);
    *reinterpret_cast<u32x4*>(dst + c * 16) = *reinterpret_cast<const u32x4*>(src + blk * 16);
    dst_s[c] = src_s[blk];
  }
}

// ------------------------------------------------------------------------------------------
// accept_prefix: chunked argmax and the prefix scan in one launch
// ------------------------------------------------------------------------------------------
// (max, lowest index) of AM_CHUNK consecutive logits of one row by a 256-thread workgroup: every
// thread issues all of its loads before merging any (one memory round trip). Thread 0 holds the
// result.
__device__ __forceinline__ void chunk_argmax(const float* r, int V, int chunk, int tid, float* sv, int* si,
                                             float& bv, int& bi) {
  const int base = chunk * AM_CHUNK;
  const int end = min(base + AM_CHUNK, V);
  bv = -INFINITY;
  bi = 0x7fffffff;
  if ((V & 3) == 0) {
    constexpr int PER = AM_CHUNK / (4 * 256);  // float4 loads per thread
    f32x4 v[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int i = base + 4 * (tid + 256 * m);
      v[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r + (i < end ? i : base)));
    }
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int i = base + 4 * (tid + 256 * m);
      if (i < end) {
        argmax_merge(bv, bi, v[m].x, i);
        argmax_merge(bv, bi, v[m].y, i + 1);
        argmax_merge(bv, bi, v[m].z, i + 2);
        argmax_merge(bv, bi, v[m].w, i + 3);
      }
    }
  } else {
    for (int i = base + tid; i < end; i += 256) argmax_merge(bv, bi, r[i], i);
  }
  wave_argmax_dpp(bv, bi);
  if ((tid & 63) == 0) { sv[tid >> 6] = bv; si[tid >> 6] = bi; }
  __syncthreads();
  if (tid == 0)
    for (int w = 1; w < 4; ++w) argmax_merge(bv, bi, sv[w], si[w]);
}

// Tag of a published chunk maximum: a 64-bit mix (the splitmix64 finaliser) of the call's epoch
// and the payload. A record whose tag matches was written by this call with exactly this payload:
// a record left by an earlier call carries that call's epoch, and a stale, garbage or partly
// written record fails the check except with probability about 2^-64.
__device__ __forceinline__ uint64_t acc_tag(uint64_t epoch, float v, int i) {
  uint64_t z = epoch ^ (((uint64_t)__float_as_uint(v) << 32) | (uint32_t)i);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Workgroup (chunk c, row y) with y = s n_target + t (sequence s, position t) takes AM_CHUNK logits
// of row y and publishes (max, index, tag) as one 16-byte device-coherent store, and is done. The
// last workgroup of each sequence (the last chunk of its last row, dispatched after every other
// workgroup of the sequence) requests all of the sequence's records at once and validates each by
// its tag, re-requesting the invalid ones until all are valid; so the records carry their own
// completion, and the workspace needs no initialisation. It then reduces each row (the merge keeps
// the maximum, ties to the lower index, so the order of the partials does not matter), and wave 0
// compares the drafts with the targets, one position per lane: the first mismatch (a ballot) is
// the accepted length. The wait is bounded: past it, accepted = -1 (the call failed). A
// sequence's draft count is n_draft, or n_draft_seq[s] clamped to [0, n_draft] when given.
// The tags mix the host's per-call epoch with a per-sequence generation word in the workspace,
// read by every workgroup at its start and advanced by the sequence's last workgroup at its end
// (after every other workgroup of the sequence has published): a launch replayed from a captured
// graph keeps its epoch argument, and the generation is what keeps an earlier replay's records
// from validating.
__global__ void __launch_bounds__(256) k_accept(const float* logits, int V, int nchunks, int n_target,
                                                const int32_t* draft, int n_draft, const int32_t* n_draft_seq,
                                                int32_t* target_ids, int32_t* accepted, u32x4* rec, uint32_t* gen,
                                                uint64_t host_epoch) {
  __shared__ float sv[4];
  __shared__ int si[4];
  __shared__ int tgt[64];
  const int chunk = blockIdx.x, y = blockIdx.y, tid = threadIdx.x;
  const int sq = y / n_target;
  const uint32_t g = gen[sq];
  const uint64_t epoch = host_epoch ^ ((uint64_t)g * 0x9E3779B97F4A7C15ull);
  const size_t nrec = (size_t)gridDim.y * nchunks;
  const rsrc_t rr = buf_rsrc(rec, (uint32_t)(nrec * 16));
  float bv;
  int bi;
  chunk_argmax(logits + (size_t)y * V, V, chunk, tid, sv, si, bv, bi);
  if (tid == 0) {
    const uint64_t t = acc_tag(epoch, bv, bi);
    const u32x4 r = {__float_as_uint(bv), (uint32_t)bi, (uint32_t)t, (uint32_t)(t >> 32)};
    __builtin_amdgcn_raw_buffer_store_b128(r, rr, (uint32_t)(((size_t)y * nchunks + chunk) * 16), 0, BUF_DEV);
  }
  if (chunk != nchunks - 1 || y % n_target != n_target - 1) return;

  // The sequence's last workgroup. Its records (row major) are taken in passes of 256 PPT, thread
  // t owning records t, t + 256, ... of a pass; each staged in LDS once valid, then each wave
  // merges rows w, w + 4, ... into the rows' running maxima (a row may span passes).
  const uint32_t r0 = (uint32_t)((size_t)sq * n_target * nchunks * 16);
  const int nf = n_target * nchunks;
  constexpr int PPT = 8;
  __shared__ float stv[256 * PPT];
  __shared__ int sti[256 * PPT];
  __shared__ float rowv[64];
  const int lane = tid & 63, wave = tid >> 6;
  int nd = n_draft;
  if (n_draft_seq) nd = min(max(n_draft_seq[sq], 0), n_draft);
  const int32_t d = (tid < nd) ? draft[(size_t)sq * n_draft + tid] : 0;  // nd <= n_target <= 64
  if (tid < 64) {
    rowv[tid] = -INFINITY;
    tgt[tid] = 0x7fffffff;
  }
  bool ok = true;
  for (int base = 0; base < nf && ok; base += 256 * PPT) {
    uint32_t seen = 0;  // bit m: record base + tid + 256 m is valid and staged
    for (uint32_t polls = 0;; ++polls) {
      u32x4 r[PPT];
#pragma unroll
      for (int m = 0; m < PPT; ++m) {
        const int i = base + tid + 256 * m;
        r[m] = (i < nf && !((seen >> m) & 1u))
                   ? __builtin_amdgcn_raw_buffer_load_b128(rr, (uint32_t)i * 16u, r0, BUF_DEV)
                   : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int m = 0; m < PPT; ++m) {
        const int i = base + tid + 256 * m;
        if (i >= nf) {
          seen |= 1u << m;
        } else if (!((seen >> m) & 1u)) {
          const float v = __uint_as_float(r[m].x);
          const uint64_t t = (uint64_t)r[m].z | ((uint64_t)r[m].w << 32);
          if (t == acc_tag(epoch, v, (int)r[m].y)) {
            stv[tid + 256 * m] = v;
            sti[tid + 256 * m] = (int)r[m].y;
            seen |= 1u << m;
          }
        }
      }
      if (__syncthreads_and(seen == (1u << PPT) - 1u)) break;
      if (polls == WAIT_POLLS) { ok = false; break; }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!ok) break;
    const int end = min(nf, base + 256 * PPT);
    if (nf <= 256 * PPT && nchunks <= 32) {
      // every record in one pass: 16 lanes per row (lane c of the row's group takes chunks c and
      // c + 16), so each wave merges four rows at once; the merge order does not change the result
      for (int rb = wave * 4; rb < n_target; rb += 16) {  // uniform over the wave
        const int row = rb + (lane >> 4), c = lane & 15;
        float v = -INFINITY;
        int vi = 0x7fffffff;
        if (row < n_target)
          for (int cc = c; cc < nchunks; cc += 16) argmax_merge(v, vi, stv[row * nchunks + cc], sti[row * nchunks + cc]);
        row16_argmax_dpp(v, vi);
        if (c == 0 && row < n_target) {
          rowv[row] = v;
          tgt[row] = vi;
        }
      }
      __syncthreads();
      break;
    }
    const int r_lo = base / nchunks, r_hi = (end - 1) / nchunks;
    for (int row = r_lo + wave; row <= r_hi; row += 4) {
      float v = rowv[row];
      int vi = tgt[row];
      const int p_lo = max(base, row * nchunks), p_hi = min(end, (row + 1) * nchunks);
      for (int i = p_lo + lane; i < p_hi; i += 64) argmax_merge(v, vi, stv[i - base], sti[i - base]);
      wave_argmax_dpp(v, vi);
      if (lane == 0) {
        rowv[row] = v;
        tgt[row] = vi;
      }
    }
    __syncthreads();  // the stage is reused by the next pass
  }
  if (!ok) {
    if (tid == 0) {
      accepted[sq] = -1;
      gen[sq] = g + 1u;
    }
    return;
  }
  if (wave == 0) {  // the rows' results are in LDS (the last pass ended with a barrier)
    const int t = tgt[lane];
    const bool miss = lane < nd && d != t;
    const unsigned long long m = __ballot(miss);
    if (lane == 0) {
      accepted[sq] = m ? __builtin_ctzll(m) : nd;
      gen[sq] = g + 1u;
    }
    if (lane < n_target) target_ids[(size_t)sq * n_target + lane] = t;
  }
}

// The output head's final pass. One workgroup of 16 waves per sequence (workgroup s: sequence s,
// its rows, drafts and results at s times the strides): wave w reduces rows w, w + 16, ... (lane l
// takes chunks l, l + 64,
// ...); then wave 0 compares the drafts with the targets, one position per lane, and the first
// mismatch (a ballot) is the accepted length. The draft ids are requested before the partials.
// A sequence's draft count is n_draft, or n_draft_seq[s] clamped to [0, n_draft] when given.
__global__ void __launch_bounds__(1024) k_accept_final(const float* pv, const int* pi, int nchunks,
                                                       int n_target, const int32_t* draft, int n_draft,
                                                       int32_t* target_ids, int32_t* accepted,
                                                       const int32_t* n_draft_seq = nullptr) {
  __shared__ int tgt[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sq = blockIdx.x;
  pv += (size_t)sq * n_target * nchunks;
  pi += (size_t)sq * n_target * nchunks;
  target_ids += (size_t)sq * n_target;
  accepted += sq;
  if (draft) draft += (size_t)sq * n_draft;
  if (n_draft_seq) n_draft = min(max(n_draft_seq[sq], 0), n_draft);
  const int32_t d = (tid < n_draft) ? draft[tid] : 0;  // n_draft <= n_target <= 64
  // The merge keeps the maximum under (value descending, index ascending), so the order in which
  // partials are merged does not change the result; the loads are issued before any merge.
  if (n_target <= 32 && nchunks <= 32) {
    // half a wave per row (rows 2w and 2w + 1 in wave w), lane c of the half takes chunk c: every
    // row in one pass
    const int row = 2 * wave + (lane >> 5), c = lane & 31;
    const size_t at = (size_t)min(row, n_target - 1) * nchunks + min(c, nchunks - 1);
    const float v = pv[at];
    const int vi = pi[at];
    const bool ok = row < n_target && c < nchunks;
    float bv = ok ? v : -INFINITY;
    int bi = ok ? vi : 0x7fffffff;
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      argmax_merge(bv, bi, ov, oi);
    }
    if (c == 0 && row < n_target) {
      tgt[row] = bi;
      target_ids[row] = bi;
    }
  } else {
    constexpr int MC = 8;  // chunks per lane loaded at once
    for (int row = wave; row < n_target; row += 16) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      const float* rv = pv + (size_t)row * nchunks;
      const int* ri = pi + (size_t)row * nchunks;
      for (int c0 = 0; c0 < nchunks; c0 += 64 * MC) {
        float v[MC];
        int vi[MC];
#pragma unroll
        for (int m = 0; m < MC; ++m) {
          const int c = c0 + lane + 64 * m;
          v[m] = rv[c < nchunks ? c : 0];
          vi[m] = ri[c < nchunks ? c : 0];
        }
#pragma unroll
        for (int m = 0; m < MC; ++m)
          if (c0 + lane + 64 * m < nchunks) argmax_merge(bv, bi, v[m], vi[m]);
      }
      wave_argmax(bv, bi);
      if (lane == 0) {
        tgt[row] = bi;
        target_ids[row] = bi;
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    const bool miss = lane < n_draft && d != tgt[lane];
    const unsigned long long m = __ballot(miss);
    if (lane == 0) accepted[0] = m ? __builtin_ctzll(m) : n_draft;
  }
}

// ------------------------------------------------------------------------------------------
// lm_head_accept: the target's output head streamed once per block, argmax fused
// ------------------------------------------------------------------------------------------
// The head is one [V x H] matrix read once for the whole block ("Speculating on a Strix Halo",
// "What the pieces cost"; "Should we shrink the vocab?"). An item is 32 head rows (two 16-row
// tiles of the tiled bf16 layout, 64 H bytes); items are scheduled as in the gate/up kernel
// (make_sched: static rounds, then the last rounds claimed from pools) with the next item's
// loads in flight while the current one is multiplied. Wave w owns H windows w WPW ..
// w WPW + WPW - 1; the block's hidden states enter MFMA as bf16 hi + lo fragments that every
// workgroup builds once. The logits never leave the chip: after the cross-wave sum each thread
// owns one fixed (tile, row, position) slot and keeps the best (logit, row) seen in it; the
// workgroup reduces its slots once at the end into one partial per position, and k_accept_final
// reduces the partials and scans the accepted prefix.
//
// No earlier kernel of the call can reset the claim pools, so each pool counter is 64-bit with
// a per-call epoch above the count: its owner (workgroup 8 p of pool p) stores (epoch, 0) when
// it starts, and a claim that returns another epoch means the pool is not set up yet and ends
// that workgroup's claiming. The owner claims until its pool is exhausted, so no item is ever
// left out whatever the workspace held; a stale counter can at worst repeat an item, which a
// maximum absorbs.
struct HeadSmem {
  float red[2][NW * 2 * 256];  // per-wave partial tiles, double-buffered across items
  float bv[NW][KMAX];
  int bi[NW][KMAX];
  int claim[4];                // ring of scheduled item indices: item h sits in claim[h % 4]
};
constexpr int HEAD_CTR_STRIDE = 32;  // uint64 words between pool counters (256 B)

// B fragments of this wave's H windows from the fp32 hidden states (bf16 K order). Every lane
// loads unconditionally (clamped to position 0 / window 0) so that all loads are in flight at
// once, then positions past n and inactive waves take zeros.
template <int WPW>
__device__ __forceinline__ void head_xb(u32x4 (&xb)[WPW][4][2], const float* h, int H, int n, int win0,
                                        bool active, int lane) {
  const int c = lane & 15, q = lane >> 4;
  const bool live = active && c < n;
  const float* row = h + (size_t)(c < n ? c : 0) * H + (active ? win0 : 0) * WIN;
  float4 v[WPW][4][2];
#pragma unroll
  for (int wi = 0; wi < WPW; ++wi)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* src = row + wi * WIN + kofs(j, q);
      v[wi][j][0] = *reinterpret_cast<const float4*>(src);
      v[wi][j][1] = *reinterpret_cast<const float4*>(src + 4);
    }
  __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the first conversion
#pragma unroll
  for (int wi = 0; wi < WPW; ++wi)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float f[8] = {v[wi][j][0].x, v[wi][j][0].y, v[wi][j][0].z, v[wi][j][0].w,
                          v[wi][j][1].x, v[wi][j][1].y, v[wi][j][1].z, v[wi][j][1].w};
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        split_bf16(f[i], hi[i], lo[i]);
        hi[i] = live ? hi[i] : 0u;
        lo[i] = live ? lo[i] : 0u;
      }
      pack8(hi, xb[wi][j][0]);
      pack8(lo, xb[wi][j][1]);
    }
}

// Cross-wave sum of one item's two tiles, then each thread's running best for its slot:
// tile tl = tid / 256, row r = 4 (p / 64) + p % 4 and position c = (p / 4) % 16 of p = tid % 256.
// Reads the item index two steps ahead from the ring after the barrier.
__device__ __forceinline__ void head_epilogue(HeadSmem& S, int buf, const f32x4 (&acc)[GU_MX_RT][2], int item,
                                              int V, int n, int wave, int lane, int tid, float& bv, int& bi,
                                              int ring, int* next) {
  float* red = S.red[buf];
  *reinterpret_cast<f32x4*>(&red[(wave * 2 + 0) * 256 + lane * 4]) = acc[0][0];
  *reinterpret_cast<f32x4*>(&red[(wave * 2 + 1) * 256 + lane * 4]) = acc[0][1];
  __syncthreads();  // one barrier per item: the other buffer takes the next item's tiles
  *next = __builtin_amdgcn_readfirstlane(S.claim[ring]);
  const int tl = tid >> 8, p = tid & 255;
  float v = 0.f;
#pragma unroll
  for (int wv = 0; wv < NW; ++wv) v += red[(wv * 2 + tl) * 256 + p];
  const int c = (p >> 2) & 15, r = 4 * (p >> 6) + (p & 3);
  const int row = item * 32 + 16 * tl + r;
  if (c < n && row < V) argmax_merge(bv, bi, v, row);
}

// item of a claimed head ticket, or n (past the end) when the ticket predates this call's epoch
__device__ __forceinline__ int head_pool_item(const Sched& q, uint64_t v, uint32_t epoch, int n) {
  const uint32_t c = (uint32_t)v;
  return ((uint32_t)(v >> 32) == epoch && c < (uint32_t)n) ? min(pool_item(q, c), n) : n;
}

template <int WPW>
__global__ void __launch_bounds__(NTH) k_head(const float* h, const uint8_t* w, int H, int V, int n,
                                              int n_items, float* pv, int* pi, uint64_t* ctr, uint32_t epoch) {
  __shared__ HeadSmem S;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = gridDim.x, b = blockIdx.x;
  const int win0 = wave * WPW;
  const bool active = win0 < H / WIN;
  const int wsafe = active ? win0 : 0;  // inactive waves load window 0 and multiply it by zero
  const uint32_t tile = (uint32_t)H * 32u;       // bytes of one 16-row tile
  const uint32_t ntile = (uint32_t)(V + 15) / 16u;
  // second-tile loads of an odd last item fall past the second resource's range and read zeros
  const rsrc_t r0 = buf_rsrc(w, ntile * tile), r1 = buf_rsrc(w + tile, (ntile - 1u) * tile);
  const uint32_t vb = (uint32_t)(256 * wsafe + lane) * 16u;
  const Sched q = make_sched(n_items, G, b, 0, nullptr);
  uint64_t* const pctr = ctr + q.pool * HEAD_CTR_STRIDE;
  if (tid == 0 && q.claims && b == 8 * q.pool)  // the pool's owner sets it up for this call
    __hip_atomic_store(pctr, (uint64_t)epoch << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  u32x4 xb[WPW][4][2];
  head_xb<WPW>(xb, h, H, n, win0, active, lane);
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  const int i0 = static_item(q, 0);
  if (i0 < n_items) {
    // step h: item h is in T[h % 2] with its loads in flight; the loads of item h + 1 are
    // issued; thread 0 stores item h + 2 into the ring (static, or claimed two steps earlier)
    // and claims item h + 4 when that one is claimed (stand-in item 0 past the end)
    GUItem<WPW> T0, T1;
    int c0 = i0, n1 = static_item(q, 1), n2;
    uint64_t ca = 0, cb = 0;
    gu_load_bf16<WPW>(T0, r0, r1, (uint32_t)c0 * 2u * tile, vb);
    for (int st = 0;; st += 2) {
      gu_load_bf16<WPW>(T1, r0, r1, (uint32_t)(n1 < n_items ? n1 : 0) * 2u * tile, vb);
      if (tid == 0) {
        S.claim[(st + 2) & 3] = is_static(q, st + 2) ? static_item(q, st + 2) : head_pool_item(q, ca, epoch, n_items);
        if (!is_static(q, st + 4))
          ca = __hip_atomic_fetch_add(pctr, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_sched_barrier(0);
      {
        f32x4 acc[GU_MX_RT][2];
        gu_math_bf16<WPW>(acc, T0, xb);
        head_epilogue(S, 0, acc, c0, V, n, wave, lane, tid, bv, bi, (st + 2) & 3, &n2);
      }
      if (n1 >= n_items) break;
      gu_load_bf16<WPW>(T0, r0, r1, (uint32_t)(n2 < n_items ? n2 : 0) * 2u * tile, vb);
      if (tid == 0) {
        S.claim[(st + 3) & 3] = is_static(q, st + 3) ? static_item(q, st + 3) : head_pool_item(q, cb, epoch, n_items);
        if (!is_static(q, st + 5))
          cb = __hip_atomic_fetch_add(pctr, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_sched_barrier(0);
      {
        f32x4 acc[GU_MX_RT][2];
        gu_math_bf16<WPW>(acc, T1, xb);
        head_epilogue(S, 1, acc, n1, V, n, wave, lane, tid, bv, bi, (st + 3) & 3, &n1);
      }
      if (n2 >= n_items) break;
      c0 = n2;
    }
  }
  // the four row slots of a position sit in lanes 4c .. 4c + 3 of each wave
#pragma unroll
  for (int off = 1; off <= 2; off <<= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    argmax_merge(bv, bi, ov, oi);
  }
  if ((lane & 3) == 0) {
    S.bv[wave][lane >> 2] = bv;
    S.bi[wave][lane >> 2] = bi;
  }
  __syncthreads();
  if (tid < n) {
    float v = S.bv[0][tid];
    int i = S.bi[0][tid];
#pragma unroll
    for (int wv = 1; wv < NW; ++wv) argmax_merge(v, i, S.bv[wv][tid], S.bi[wv][tid]);
    pv[(size_t)tid * G + b] = v;
    pi[(size_t)tid * G + b] = i;
  }
}

// ------------------------------------------------------------------------------------------
// accept_sample: lossless acceptance at temperature T, and acceptance statistics
// ------------------------------------------------------------------------------------------
// The committed tokens are distributed exactly as the target's own samples at any temperature
// ("Speculating on a Strix Halo", "Speculative decoding", whose reference 2 gives the rule):
// with p_i = softmax(target_i / T) and q_i = softmax(draft_i / T), draft d_i is kept while
// u_accept[i] q_i(d_i) < p_i(d_i); at the first rejection a the token is drawn from the
// renormalised residual max(0, p_a - q_a) (p_a itself if that has no mass); when every draft is
// kept, from p_n. Logits are scaled to base-2 exponents z = l log2(e) / T once.
//   k_lse_partial     (chunk, row): chunk maximum and sum of 2^(z - max), target and draft rows
//   k_sample_partial  chunk c: every workgroup merges the row partials and takes the accept
//                     decisions (identical data and code, so identical results); then the weights
//                     of its chunk of the row to sample are summed with the fixed-order block scan
//   k_sample_final    one workgroup: the chunk whose running total first exceeds u W, then the
//                     element inside it, with the same scan, so the chunk totals agree bit for bit
constexpr int SAMPLE_NTH = 1024;  // threads of the sampling workgroups: 8 values each per chunk
static_assert(SAMPLE_NTH * 8 == AM_CHUNK, "one chunk per sampling workgroup");
enum { SAMPLE_NONE = 0, SAMPLE_RESIDUAL = 1, SAMPLE_TARGET = 2 };
struct SamplePlan {
  int a, mode, row, pad;
  float mt, st, md, sd, u;
};

// (max, sum) pairs of 2^(z - max) partial sums, combined; an empty side (max -inf) adds nothing
__device__ __forceinline__ void lse_merge(float& m, float& s, float mo, float so) {
  const float mm = fmaxf(m, mo);
  if (mm == -INFINITY) return;
  s = (m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f(m - mm)) +
      (mo == -INFINITY ? 0.f : so * __builtin_amdgcn_exp2f(mo - mm));
  m = mm;
}
// DPP lane moves of fp32 values (CTRL: the DPP control; lanes outside ROWMASK keep 0)
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWMASK, 0xf, true));
}
// Wave-uniform maximum and sum over the 64 lanes (every lane of a 16-lane row gets the row result
// from four full-row permutations, then the four row results in a fixed order).
__device__ __forceinline__ float wave_max_f32(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f32<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f32<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_f32<0x140>(x));  // row_mirror
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)),
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)),
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48))));
}
__device__ __forceinline__ float wave_sum_f32(float x) {
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x141>(x);
  x += dpp_f32<0x140>(x);
  return (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48)));
}
// wave-uniform merge of the lanes' (max, sum) pairs: the maximum first, then one rescale per lane
__device__ __forceinline__ void wave_lse(float& m, float& s) {
  const float mm = wave_max_f32(m);
  const float t = (m == -INFINITY) ? 0.f : s * __builtin_amdgcn_exp2f(m - mm);
  s = wave_sum_f32(t);
  m = mm;
}

__global__ void __launch_bounds__(256) k_lse_partial(const float* tl, const float* dl, int n_t, int V, int nchunks,
                                                     float zscale, float2* ms) {
  __shared__ float sm[4], ss[4];
  const int row = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  {  // sequence blockIdx.z of a batch: its rows and partials
    const int sq = blockIdx.z, n_d = gridDim.y - n_t;
    tl += (size_t)sq * n_t * V;
    dl += (size_t)sq * n_d * V;
    ms += (size_t)sq * gridDim.y * nchunks;
  }
  const float* r = row < n_t ? tl + (size_t)row * V : dl + (size_t)(row - n_t) * V;
  const int base = chunk * AM_CHUNK, end = min(base + AM_CHUNK, V);
  constexpr int PER = AM_CHUNK / (4 * 256);
  float z[PER * 4];
  if ((V & 3) == 0) {
    f32x4 v[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int i = base + 4 * (tid + 256 * m);
      v[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r + (i < end ? i : base)));
    }
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int i = base + 4 * (tid + 256 * m);
      const float e[4] = {v[m].x, v[m].y, v[m].z, v[m].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) z[4 * m + j] = (i + j < end) ? e[j] * zscale : -INFINITY;
    }
  } else {
#pragma unroll
    for (int m = 0; m < PER; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = base + 4 * (tid + 256 * m) + j;
        z[4 * m + j] = i < end ? r[i] * zscale : -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER * 4; ++i) mx = fmaxf(mx, z[i]);
  float sum = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int i = 0; i < PER * 4; ++i) sum += __builtin_amdgcn_exp2f(z[i] - mx);
  }
  wave_lse(mx, sum);
  if ((tid & 63) == 0) { sm[tid >> 6] = mx; ss[tid >> 6] = sum; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) lse_merge(mx, sum, sm[w], ss[w]);
    ms[(size_t)row * nchunks + chunk] = make_float2(mx, sum);
  }
}

// Inclusive prefix sums of one value per thread over the 1024 threads, in a fixed order (wave
// scans, then the wave totals scanned by one wave); every caller sees identical bits for
// identical inputs.
__device__ __forceinline__ float wave_scan_incl(float v, int lane) {
  (void)lane;
  v += dpp_f32<0x111>(v);       // row_shr:1 (lanes without a source add 0)
  v += dpp_f32<0x112>(v);       // row_shr:2
  v += dpp_f32<0x114>(v);       // row_shr:4
  v += dpp_f32<0x118>(v);       // row_shr:8: inclusive scans of each 16-lane row
  v += dpp_f32<0x142, 0xa>(v);  // row_bcast:15: row 0's total into row 1, row 2's into row 3
  v += dpp_f32<0x143, 0xc>(v);  // row_bcast:31: the total of rows 0-1 into rows 2 and 3
  return v;
}
__device__ __forceinline__ float block_scan_1024(float v, float* lds16, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  v = wave_scan_incl(v, lane);
  if (lane == 63) lds16[wave] = v;
  __syncthreads();
  if (wave == 0) {
    float t = lane < 16 ? lds16[lane] : 0.f;
    t = wave_scan_incl(t, lane);
    const float ex = __shfl_up(t, 1);
    if (lane < 16) lds16[16 + lane] = lane ? ex : 0.f;  // totals of the earlier waves
  }
  __syncthreads();
  const float before = lds16[16 + wave];
  __syncthreads();  // lds16 may be rewritten by the next scan
  return before + v;
}

struct SampleSmem {
  float m[128], s[128];  // merged (max, sum) per row: target rows, then draft rows
  float scan[32];
  SamplePlan plan;
  int best;
};

// Loads of the 8 consecutive elements 8t .. 8t+7 of chunk c of one row (clamped past V).
__device__ __forceinline__ void load8(const float* row, int V, int x0, float (&v)[8]) {
  if ((V & 3) == 0 && x0 + 8 <= V) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(row + x0);
    const f32x4 b = *reinterpret_cast<const f32x4*>(row + x0 + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = row[x0 + j < V ? x0 + j : 0];
  }
}

// The weights of chunk c of the plan's row, thread t holding elements 8t .. 8t+7 of the chunk:
// residual max(0, p - q) (w) and target p (p); elements past V weigh zero.
__device__ __forceinline__ void sample_weights(const float* tl, const float* dl, int V, float zscale,
                                               const SamplePlan& P, int c, int tid, float (&w)[8], float (&p)[8]) {
  const int x0 = c * AM_CHUNK + 8 * tid;
  const bool res = P.mode == SAMPLE_RESIDUAL;
  const float* rt = tl + (size_t)P.row * V;
  const float* rd = res ? dl + (size_t)P.row * V : rt;  // a target row stands in when unused
  float lt[8], ld[8];
  load8(rt, V, x0, lt);
  load8(rd, V, x0, ld);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool in = x0 + j < V;
    const float pt = in ? __builtin_amdgcn_exp2f(lt[j] * zscale - P.mt) / P.st : 0.f;
    const float pd = (in && res) ? __builtin_amdgcn_exp2f(ld[j] * zscale - P.md) / P.sd : 0.f;
    p[j] = pt;
    w[j] = fmaxf(pt - pd, 0.f);
  }
}

// Merge the row partials, take the accept decisions, and fill the plan (every workgroup alike).
// The logits at the drafted ids and every row's partials are requested together.
__device__ void sample_plan(const float* tl, const float* dl, int n_t, int V, int nchunks, float zscale,
                            const int32_t* draft, int n_d, const float* u_acc, const float* u_smp,
                            const float2* ms, SampleSmem& S, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const int R = n_t + n_d;
  // wave 0: the drafted ids' logits (lane i < n_d)
  float lt_d = 0.f, ld_d = 0.f, ua = 0.f;
  bool valid = false;
  if (wave == 0 && lane < n_d) {
    const int d = draft[lane];
    valid = d >= 0 && d < V;
    const int dd = valid ? d : 0;
    lt_d = tl[(size_t)lane * V + dd];
    ld_d = dl[(size_t)lane * V + dd];
    ua = u_acc[lane];
  }
  // every wave: rows wave, wave + 16, ... (at most 8), chunks lane, lane + 64, ...
  constexpr int RPW = 128 / (SAMPLE_NTH / 64);
  float2 v[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int row = min(wave + 16 * j, R - 1), c = min(lane, nchunks - 1);
    v[j] = ms[(size_t)row * nchunks + c];
  }
  float m[RPW], sm[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const bool live = wave + 16 * j < R && lane < nchunks;
    m[j] = live ? v[j].x : -INFINITY;
    sm[j] = live ? v[j].y : 0.f;
  }
  for (int c = lane + 64; c < nchunks; c += 64)  // vocabularies beyond 64 chunks
#pragma unroll
    for (int j = 0; j < RPW; ++j)
      if (wave + 16 * j < R) {
        const float2 o = ms[(size_t)(wave + 16 * j) * nchunks + c];
        lse_merge(m[j], sm[j], o.x, o.y);
      }
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    wave_lse(m[j], sm[j]);
    if (lane == 0 && wave + 16 * j < R) { S.m[wave + 16 * j] = m[j]; S.s[wave + 16 * j] = sm[j]; }
  }
  __syncthreads();
  if (wave == 0) {
    bool miss = false;
    if (lane < n_d) {
      const float p = __builtin_amdgcn_exp2f(lt_d * zscale - S.m[lane]) / S.s[lane];
      const float q = __builtin_amdgcn_exp2f(ld_d * zscale - S.m[n_t + lane]) / S.s[n_t + lane];
      miss = !(valid && ua * q < p);
    }
    const unsigned long long mm = __ballot(miss);
    if (lane == 0) {
      SamplePlan P;
      P.a = mm ? __builtin_ctzll(mm) : n_d;
      P.pad = 0;
      if (P.a < n_d) { P.mode = SAMPLE_RESIDUAL; P.row = P.a; }
      else if (n_d < n_t) { P.mode = SAMPLE_TARGET; P.row = n_d; }
      else { P.mode = SAMPLE_NONE; P.row = 0; }
      P.mt = S.m[P.row]; P.st = S.s[P.row];
      P.md = P.mode == SAMPLE_RESIDUAL ? S.m[n_t + P.row] : 0.f;
      P.sd = P.mode == SAMPLE_RESIDUAL ? S.s[n_t + P.row] : 1.f;
      P.u = P.mode == SAMPLE_NONE ? 0.f : u_smp[P.row];
      S.plan = P;
    }
  }
  __syncthreads();
}

__global__ void __launch_bounds__(SAMPLE_NTH) k_sample_partial(const float* tl, const float* dl, int n_t, int V,
                                                               int nchunks, float zscale, const int32_t* draft,
                                                               int n_d, const float* u_acc, const float* u_smp,
                                                               const float2* ms, float2* csum, SamplePlan* plan,
                                                               int32_t* accepted, int32_t* token) {
  __shared__ SampleSmem S;
  const int tid = threadIdx.x, c = blockIdx.x;
  {  // sequence blockIdx.y of a batch
    const size_t sq = blockIdx.y;
    tl += sq * n_t * V;
    dl += sq * n_d * V;
    draft += sq * n_d;
    u_acc += sq * n_d;
    u_smp += sq * n_t;
    ms += sq * (n_t + n_d) * nchunks;
    csum += sq * nchunks;
    plan += sq;
    accepted += sq;
    token += sq;
  }
  sample_plan(tl, dl, n_t, V, nchunks, zscale, draft, n_d, u_acc, u_smp, ms, S, tid);
  const SamplePlan P = S.plan;
  if (c == 0 && tid == 0) {
    *plan = P;
    accepted[0] = P.a;
    if (P.mode == SAMPLE_NONE) token[0] = -1;
  }
  if (P.mode == SAMPLE_NONE) return;  // uniform across the grid
  float w[8], p[8];
  sample_weights(tl, dl, V, zscale, P, c, tid, w, p);
  float tw = 0.f, tp = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) { tw += w[j]; tp += p[j]; }
  const float sw = block_scan_1024(tw, S.scan, tid);
  const float sp = block_scan_1024(tp, S.scan, tid);
  if (tid == SAMPLE_NTH - 1) csum[c] = make_float2(sw, sp);
}

__global__ void __launch_bounds__(SAMPLE_NTH) k_sample_final(const float* tl, const float* dl, int V, int nchunks,
                                                             float zscale, const float2* csum, const SamplePlan* plan,
                                                             int32_t* token, int n_t = 0, int n_d = 0) {
  __shared__ SampleSmem S;
  __shared__ int sel_chunk, use_res, lastw;
  __shared__ float sel_base, sel_target;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  {  // sequence blockIdx.x of a batch (n_t, n_d: its target and draft row counts)
    const size_t sq = blockIdx.x;
    tl += sq * n_t * V;
    dl += sq * n_d * V;
    csum += sq * nchunks;
    plan += sq;
    token += sq;
  }
  const SamplePlan P = *plan;
  if (P.mode == SAMPLE_NONE) return;
  if (wave == 0) {
    // residual chunk totals unless they have no mass; running totals by a wave scan per 64 chunks
    float totw = 0.f;
    for (int c0 = 0; c0 < nchunks; c0 += 64) {
      const float x = c0 + lane < nchunks ? csum[c0 + lane].x : 0.f;
      totw += __shfl(wave_scan_incl(x, lane), 63);
    }
    const bool res = P.mode == SAMPLE_RESIDUAL && totw > 0.f;
    float tot = 0.f;
    for (int c0 = 0; c0 < nchunks; c0 += 64) {
      const float2 cv = c0 + lane < nchunks ? csum[c0 + lane] : make_float2(0.f, 0.f);
      tot += __shfl(wave_scan_incl(res ? cv.x : cv.y, lane), 63);
    }
    const float target = P.u * tot;
    int sel = -1, last = -1;
    float base = 0.f, lastbase = 0.f, run = 0.f;
    for (int c0 = 0; c0 < nchunks && sel < 0; c0 += 64) {
      const float2 cv = c0 + lane < nchunks ? csum[c0 + lane] : make_float2(0.f, 0.f);
      const float wc = res ? cv.x : cv.y;
      const float incl = run + wave_scan_incl(wc, lane);
      const float excl = incl - wc;
      const unsigned long long cross = __ballot(wc > 0.f && incl > target);
      const unsigned long long nz = __ballot(wc > 0.f);
      if (cross) {
        const int l = __builtin_ctzll(cross);
        sel = c0 + l;
        base = __shfl(excl, l);
      }
      if (nz) {
        const int l = 63 - __builtin_clzll(nz);
        last = c0 + l;
        lastbase = __shfl(excl, l);
      }
      run = __shfl(incl, 63);
    }
    if (sel < 0) { sel = last; base = lastbase; }  // u at or past the top: the last weighted chunk
    if (lane == 0) {
      sel_chunk = sel;
      sel_base = base;
      sel_target = target;
      use_res = res;
      S.best = 0x7fffffff;
      lastw = -1;
    }
  }
  __syncthreads();
  const int c = sel_chunk;
  float w[8], p[8];
  sample_weights(tl, dl, V, zscale, P, c, tid, w, p);
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = use_res ? w[j] : p[j];
  float tv = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) tv += v[j];
  const float incl = block_scan_1024(tv, S.scan, tid);
  const float target = sel_target;
  int first = 0x7fffffff, lastnz = -1;
  float run = sel_base + (incl - tv);  // running total before this thread's elements
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    run += v[j];
    if (v[j] > 0.f) lastnz = j;
    if (first == 0x7fffffff && v[j] > 0.f && run > target) first = j;
  }
  const int x0 = c * AM_CHUNK + 8 * tid;
  if (first != 0x7fffffff) atomicMin(&S.best, x0 + first);
  if (lastnz >= 0) atomicMax(&lastw, x0 + lastnz);
  __syncthreads();
  // no crossing inside the chunk (rounding at its top): its last weighted element
  if (tid == 0) token[0] = S.best != 0x7fffffff ? S.best : lastw;
}

// Cycle statistics: hist[j] = cycles that accepted exactly j drafts, survival[i] = cycles that
// accepted at least i + 1 (values outside [0, n_draft] are not counted). One workgroup.
__global__ void __launch_bounds__(1024) k_accept_hist(const int32_t* acc, int n_cycles, int n_draft, int64_t* hist,
                                                      int64_t* survival) {
  __shared__ unsigned long long h[65];
  const int tid = threadIdx.x;
  if (tid <= n_draft) h[tid] = 0ull;
  __syncthreads();
  for (int i = tid; i < n_cycles; i += 1024) {
    const int a = acc[i];
    if (a >= 0 && a <= n_draft) atomicAdd(&h[a], 1ull);
  }
  __syncthreads();
  if (tid <= n_draft) hist[tid] = (int64_t)h[tid];
  if (tid < n_draft) {
    unsigned long long sv = 0;
    for (int j = tid + 1; j <= n_draft; ++j) sv += h[j];
    survival[tid] = (int64_t)sv;
  }
}

// ------------------------------------------------------------------------------------------
// Gathered path: many sequences verified together (up to BT_MAX tokens per call). Each token
// still routes on its own ("Speculating on a Strix Halo", section "What the pieces cost"), but
// with hundreds of tokens nearly every expert wakes, each for a few dozen of them, so the
// experts' B operands become per-expert token gathers (tokens sorted by expert, "Speculating on
// a Strix Halo", section "The verify's own cost"):
//
//   k_brouter   (64-token, 64-expert, column slice) workgroups, fp32 MFMA over LDS-staged rows:
//               partial logits and sums of squares per slice, and each token's bf16 hi/lo B
//               fragments (token-major).
//   k_btopk     one wave per token: the slice partials added in slice order, the RMSNorm factor,
//               top-K (ties to the lower expert), softmax over the K.
//   k_bperm     eight workgroups, each: per-expert token bitmasks (LDS), counts, a scan over
//               experts for the list offsets and item counts, then the list position of each
//               (token, slot) pair of one eighth of the experts = expert offset + number of the
//               expert's tokens below it. The list (tokens by expert, then token) is
//               deterministic; the shared expert follows as slot U with every token.
//   k_bexp<GU>  (woken slot u, column group, row block) items over a flat sequence of window
//               ticks. Per tick every wave streams two 16-row A bands (gate + up rows of one
//               tile, or two row tiles of down) of one window (bf16) or two (mxfp4); the item's
//               gathered token columns for that tick are loaded by all threads and staged
//               through a two-slot LDS ring. Weights are requested two ticks ahead; the gate/up
//               epilogue fuses the reduction, SwiGLU with the RMSNorm factor and the routing
//               weight, and stores the down B operands per list position; the down epilogue
//               stores fp32 partial rows per list position. mxfp4 layers run the bf16 shared
//               expert's items first, then the routed experts' mxfp4 items, in the same launch.
//   k_bcombine  y[t] = sum_j P[pos(t, j)] + P[shared(t)] (+ x[t]), fixed slot order.
// ------------------------------------------------------------------------------------------
constexpr int BT_MAX = 1024;      // tokens per gathered call
constexpr int BTW = BT_MAX / 32;  // token-mask words per expert
constexpr int BCG = 2;            // 16-token column tiles per gathered item
constexpr int BD = 3;             // weight ticks in flight (loads issued BD - 1 ticks ahead)
constexpr int BPERM_NTH = 1024;
constexpr int BPERM_G = 8;        // permutation workgroups (each places the pairs of 1/8 of the experts)

struct BArgs {
  const float* x;
  float* y;
  int32_t* out_ids;
  float* out_w;
  int32_t* out_n;
  const float* wr;
  const uint8_t* wg;
  const uint8_t* wu;
  const uint8_t* wd;
  const uint8_t* shg;
  const uint8_t* shu;
  const uint8_t* shd;
  const uint8_t* sg;  // mxfp4 scales of the routed experts (NULL for bf16 layers)
  const uint8_t* su;
  const uint8_t* sd;
  float* logits;    // [H / gr_slice(H)][T][E] partial raw router logits of each column slice
  float* psq;       // [H / gr_slice(H)][T] partial sums of squares of each column slice
  float* rinv;      // [T] RMSNorm factor (1 without pre-norm)
  uint8_t* xg;      // [T][H/128][512 B] bf16 hi/lo B fragments of each token, k-step j, half hl,
                    // lane quad q at ((j * 2 + hl) * 4 + q) * 16
  int32_t* ids;     // [T][K]
  float* wts;       // [T][K]
  int32_t* tab;     // [0] U, [1] gate/up items, [2] down items (the kernels read [0]; the item
                    // counts are also the last entries of the prefixes below)
  int32_t* ut;      // 5 arrays of E + 2: slot u -> expert (-1: shared), list offset, count,
                    // gate/up item prefix, down item prefix (entry U + 1: totals)
  int32_t* blist;   // [T K + T] token at list position p (positions T K + t: the shared expert)
  float* bw;        // [T K + T] routing weight at position p (1 for the shared expert)
  float* brv;       // [T K + T] RMSNorm factor of the token at position p
  int32_t* bpos;    // [T][K] list position of (token, slot)
  uint8_t* af;      // [(T K + T + 16)][I/128][512 B] down B operands per list position
  uint8_t* xgm;     // mxfp4 layers: [T][H/128][MXT] MX-fp8 hi/lo B windows of each token (else NULL)
  uint8_t* afm;     // mxfp4 layers: [(T K + T + 16)][I/128][MXT] down B windows per list position
  float* part;      // [T K + T][H] fp32 partial rows per list position
  int H, E, K, I, Is, T, pre_norm, residual;
  float eps;
};

__device__ __forceinline__ int* ut_arr(const BArgs& a, int which) { return a.ut + which * (a.E + 2); }

// Token-major MX-fp8 window of one column (128 values, mxfp4 layers): hi [4 lane quads][32 B] and
// lo [4][32 B] in the scaled instruction's B-lane byte order (quad q holds K = 16 q + j in bytes
// j < 16 and K = 64 + 16 q + j in bytes 16 + j), then the scale words of the four 32-blocks (hi
// exponent in byte 0, lo in byte 1): the column's share of an MXW window, contiguous.
constexpr int MXT = 272;
__device__ __forceinline__ void mx8_store16_tok(uint8_t* tw, int blk, int h, const uint32_t (&hi)[4],
                                                const uint32_t (&lo)[4], int eh, int el) {
  const int q = 2 * (blk & 1) + h, off = 16 * (blk >> 1);
  *reinterpret_cast<u32x4*>(tw + q * 32 + off) = u32x4{hi[0], hi[1], hi[2], hi[3]};
  *reinterpret_cast<u32x4*>(tw + 128 + q * 32 + off) = u32x4{lo[0], lo[1], lo[2], lo[3]};
  if (h == 0)
    *reinterpret_cast<uint32_t*>(tw + 256 + 4 * blk) = (uint32_t)(eh + 127) | ((uint32_t)(el + 127) << 8);
}

// The many-token router is an fp32 [T x H] x [H x E] product on fp32 MFMA (16 x 16 x 4), split
// over the columns: workgroup (64-token group, 64-expert group, column slice of gr_slice(H)) stages
// its slice of the token rows and router rows in LDS, each row in contiguous 256-byte pieces (64
// columns per chunk, every load of the slice issued at once), and each of its 16 waves takes one
// 16 x 16 (expert, token) tile over the slice, lane (row r = lane % 16, quad q = lane / 16) reading
// columns 16 g + 4 q .. 16 g + 4 q + 3 of expert row r and of token row r (the same k order for both
// operands). Reading each operand piece from the cache once per workgroup, instead of once per
// wave and tile, is what lets the matrix cores set the pace. The partial logits [slice][T][E] and
// partial sums of squares [slice][T] are added by k_btopk in slice order, and the slice width
// depends only on H, so a token's logits are summed in the same order whatever the call. The same
// LDS rows give the tokens' bf16 hi/lo B fragments and (mxfp4 layers) MX-fp8 windows.
constexpr int BR_NW = 16, BR_NTH = 64 * BR_NW;
constexpr int GR_T = 64, GR_E = 64, GR_KC = 64, GR_LD = GR_KC + 4;  // LDS rows padded by 16 bytes
__host__ __device__ constexpr int gr_slice(int H) { return H % 256 == 0 ? 256 : 128; }
constexpr int GR_MS = 8;  // slices at most: H <= 2048 in 256-column slices, or H <= 896 in 128-column ones

template <int NCH>
struct alignas(16) BRouterSmem {
  float x[NCH][GR_T][GR_LD];
  float w[NCH][GR_E][GR_LD];
};

template <int NCH>
__global__ void __launch_bounds__(BR_NTH) k_brouter(BArgs a) {
  __shared__ BRouterSmem<NCH> S;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, E = a.E, T = a.T;
  constexpr int SW = NCH * GR_KC;
  const int ns = H / SW, neg = (E + GR_E - 1) / GR_E;
  const int b = blockIdx.x;
  const int sl = b % ns, eg = (b / ns) % neg, tg = b / (ns * neg);
  const int t0 = tg * GR_T, e0 = eg * GR_E, c0 = sl * SW;
  // thread: row tid / 16 of the chunk's token rows and router rows, 16-byte piece tid % 16;
  // rows past T or E read the last row (their results are never stored)
  const int lr = tid >> 4, lc = (tid & 15) * 4;
  const float* xr = a.x + (size_t)min(t0 + lr, T - 1) * H + c0 + lc;
  const float* wr = a.wr + (size_t)min(e0 + lr, E - 1) * H + c0 + lc;
  f32x4 vx[NCH], vw[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    vx[c] = *reinterpret_cast<const f32x4*>(xr + c * GR_KC);
    vw[c] = *reinterpret_cast<const f32x4*>(wr + c * GR_KC);
  }
  const int tt = wave & 3, et = wave >> 2, r = lane & 15, q = lane >> 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    *reinterpret_cast<f32x4*>(&S.x[c][lr][lc]) = vx[c];
    *reinterpret_cast<f32x4*>(&S.w[c][lr][lc]) = vw[c];
    __syncthreads();  // chunk c is complete; later chunks use other rows of LDS
    f32x4 av[GR_KC / 16], bv[GR_KC / 16];  // the chunk's operands, read before its first MFMA
#pragma unroll
    for (int g = 0; g < GR_KC / 16; ++g) {
      av[g] = *reinterpret_cast<const f32x4*>(&S.w[c][et * 16 + r][16 * g + 4 * q]);
      bv[g] = *reinterpret_cast<const f32x4*>(&S.x[c][tt * 16 + r][16 * g + 4 * q]);
    }
#pragma unroll
    for (int g = 0; g < GR_KC / 16; ++g) {
      ss += bv[g][0] * bv[g][0] + bv[g][1] * bv[g][1] + bv[g][2] * bv[g][2] + bv[g][3] * bv[g][3];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[g][j], bv[g][j], acc, 0, 0, 0);
    }
  }
  {  // D[i][j] in lane j + 16 (i / 4), element i % 4: expert e0 + 16 et + i, token t0 + 16 tt + j
    const int t = t0 + tt * 16 + r, e = e0 + et * 16 + 4 * q;
    float* pl = a.logits + ((size_t)sl * T + (t < T ? t : 0)) * E + e;
    if (E % 4 == 0) {
      if (t < T && e < E) *reinterpret_cast<f32x4*>(pl) = acc;
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (t < T && e + v < E) pl[v] = acc[v];
    }
  }
  if (eg == 0 && et == 0) {  // the slice's sum of squares of token 16 tt + r: its four quads' sums
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const int t = t0 + tt * 16 + r;
    if (q == 0 && t < T) a.psq[(size_t)sl * T + t] = ss;
  }
  // B fragments of the group's tokens in the slice: units (window wi, token tile tt) = u, wi = u / 4,
  // dealt over the token group's expert-group workgroups (unit u to eg = u mod neg), 256 threads
  // per unit (token, k-step and lane quad of tid % 256)
  const int nwt = H / WIN, nws = SW / WIN;
  for (int u = eg + neg * (tid >> 8); u < 4 * nws; u += neg * (BR_NTH / 256)) {
    const int wi = u >> 2, rr = tid & 255, tc = (u & 3) * 16 + (rr & 15), j = (rr >> 4) & 3, qq = rr >> 6;
    const int tok = t0 + tc;
    const int col = wi * WIN + kofs(j, qq);  // within the slice: chunk col / 64, 8 values
    const float* src = &S.x[col / GR_KC][tc][col % GR_KC];
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4);
    const float f[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) split_bf16(f[i], hi[i], lo[i]);
    u32x4 hv, lv;
    pack8(hi, hv);
    pack8(lo, lv);
    if (tok < T) {
      uint8_t* dst = a.xg + ((size_t)tok * nwt + sl * nws + wi) * 512;
      *reinterpret_cast<u32x4*>(dst + ((j * 2 + 0) * 4 + qq) * 16) = hv;
      *reinterpret_cast<u32x4*>(dst + ((j * 2 + 1) * 4 + qq) * 16) = lv;
    }
  }
  // mxfp4 layers: the MX-fp8 windows of the routed experts' B operands, one wave per unit (window
  // wi, token tile tt) = u as above, lane (column c, 32-block blk)
  if (a.xgm) {
    const int c = lane & 15, blk = lane >> 4;
    for (int u = eg + neg * wave; u < 4 * nws; u += neg * BR_NW) {
      const int wi = u >> 2, tc = (u & 3) * 16 + c, tok = t0 + tc;
      const int col = wi * WIN + 32 * blk;
      const float* src = &S.x[col / GR_KC][tc][col % GR_KC];
      float v[32];
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const f32x4 f = *reinterpret_cast<const f32x4*>(src + 4 * g);
        v[4 * g + 0] = f[0]; v[4 * g + 1] = f[1]; v[4 * g + 2] = f[2]; v[4 * g + 3] = f[3];
      }
      uint32_t hi[8], lo[8];
      int eh, el;
      mx8_quant<32, false>(v, hi, lo, eh, el);
      if (tok < T) {
        uint8_t* tw = a.xgm + ((size_t)tok * nwt + sl * nws + wi) * MXT;
        const uint32_t h0[4] = {hi[0], hi[1], hi[2], hi[3]}, h1[4] = {hi[4], hi[5], hi[6], hi[7]};
        const uint32_t l0[4] = {lo[0], lo[1], lo[2], lo[3]}, l1[4] = {lo[4], lo[5], lo[6], lo[7]};
        mx8_store16_tok(tw, blk, 0, h0, l0, eh, el);
        mx8_store16_tok(tw, blk, 1, h1, l1, eh, el);
      }
    }
  }
}

// A lane's NS logits (experts e0 ..) as the sum of the router's ns slice partials, slice 0 first;
// every slice's loads are issued before the first add
template <int NS>
__device__ __forceinline__ void slice_logits(const float* row, size_t stride, int ns, int e0, int E, float (&v)[NS]) {
  float p[GR_MS][NS];
#pragma unroll
  for (int sl = 0; sl < GR_MS; ++sl) lane_logits<NS>(row + (sl < ns ? sl : ns - 1) * stride, e0, E, p[sl]);
#pragma unroll
  for (int m = 0; m < NS; ++m) v[m] = p[0][m];
#pragma unroll
  for (int sl = 1; sl < GR_MS; ++sl)
    if (sl < ns)
#pragma unroll
      for (int m = 0; m < NS; ++m) v[m] += p[sl][m];
}

// one wave per token: its logits and sum of squares from the router's slice partials (slice
// order), the RMSNorm factor, top-K over the scaled logits, softmax over the K
__global__ void __launch_bounds__(NTH) k_btopk(BArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * NW + (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= a.T) return;
  const int E = a.E, K = a.K, T = a.T;
  const int ns = a.H / gr_slice(a.H);  // the router's column slices, added in slice order
  float pq[GR_MS];
#pragma unroll
  for (int sl = 0; sl < GR_MS; ++sl) pq[sl] = a.psq[(size_t)(sl < ns ? sl : ns - 1) * T + t];
  float sq = pq[0];
#pragma unroll
  for (int sl = 1; sl < GR_MS; ++sl)
    if (sl < ns) sq += pq[sl];
  const float rv = a.pre_norm ? 1.0f / sqrtf(sq / (float)a.H + a.eps) : 1.0f;
  if (lane == 0) a.rinv[t] = rv;
  const float* lg = a.logits + (size_t)t * E;
  const size_t lst = (size_t)T * E;  // between the slices' partial rows
  int my_e = 0;
  uint32_t my_key = 0;
  if (E <= 256) {  // experts 4 lane + m
    float v[4];
    slice_logits<4>(lg, lst, ns, 4 * lane, E, v);
    uint64_t c[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = 4 * lane + m;
      c[m] = topk_comp(e < E ? okey32(rv * v[m]) : 0u, e);
    }
    sort_desc<4>(c);
    topk_sorted<4, false>(c, K, lane, my_e, my_key);
  } else {  // experts 8 lane + m
    float v[8];
    slice_logits<8>(lg, lst, ns, 8 * lane, E, v);
    uint64_t c[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int e = 8 * lane + m;
      c[m] = topk_comp(e < E ? okey32(rv * v[m]) : 0u, e);
    }
    sort_desc<8>(c);
    topk_sorted<8, false>(c, K, lane, my_e, my_key);
  }
  const float my_val = okey32_value(my_key);
  const float m0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_val), 0));
  const float ex = expf(my_val - m0);
  float sum = 0.f;
  for (int j = 0; j < K; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
  if (lane < K) {
    const float w = ex / sum;
    a.ids[t * K + lane] = my_e;
    a.wts[t * K + lane] = w;
    if (a.out_ids) a.out_ids[t * K + lane] = my_e;
    if (a.out_w) a.out_w[t * K + lane] = w;
  }
}

// exclusive prefix over the workgroup's threads (BPERM_NTH) of four counters at once; tot gets
// the sums
__device__ __forceinline__ int4 block_excl_scan4(int4 v, int4* wsum, int tid, int4& tot) {
  const int lane = tid & 63, wave = tid >> 6;
  int4 inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ax = __shfl_up(inc.x, o), ay = __shfl_up(inc.y, o), az = __shfl_up(inc.z, o),
              aw = __shfl_up(inc.w, o);
    if (lane >= o) { inc.x += ax; inc.y += ay; inc.z += az; inc.w += aw; }
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int4 base = {0, 0, 0, 0};
  tot = base;
  for (int w = 0; w < BPERM_NTH / 64; ++w) {
    const int4 s = wsum[w];
    if (w < wave) { base.x += s.x; base.y += s.y; base.z += s.z; base.w += s.w; }
    tot.x += s.x; tot.y += s.y; tot.z += s.z; tot.w += s.w;
  }
  return int4{base.x + inc.x - v.x, base.y + inc.y - v.y, base.z + inc.z - v.z, base.w + inc.w - v.w};
}

struct PermSmem {
  uint32_t msk[MAX_E * BTW];
  uint16_t wpre[MAX_E * BTW];  // the expert's tokens in the words before this one
  int eoff[MAX_E];
  int4 wsum[BPERM_NTH / 64];
};

__global__ void __launch_bounds__(BPERM_NTH) k_bperm(BArgs a) {
  __shared__ PermSmem S;
  constexpr int PPT = BT_MAX * MAX_K / BPERM_NTH;  // (token, slot) pairs per thread at most
  const int tid = threadIdx.x;
  const int T = a.T, E = a.E, K = a.K, H = a.H;
  const int tw = (T + 31) / 32, n = T * K;
  // the thread's pairs i = tid + BPERM_NTH m, all requested at once (one memory round trip)
  const int g = blockIdx.x, ng = gridDim.x;
  int pte[PPT];  // token << 16 | expert
#pragma unroll
  for (int m = 0; m < PPT; ++m) {
    const int i = tid + BPERM_NTH * m;
    const int ic = i < n ? i : 0;
    pte[m] = ((ic / K) << 16) | a.ids[ic];
  }
  for (int i = tid; i < E * tw; i += BPERM_NTH) S.msk[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int m = 0; m < PPT; ++m)
    if (tid + BPERM_NTH * m < n) {
      const int t = pte[m] >> 16, e = pte[m] & 0xFFFF;
      atomicOr(&S.msk[e * tw + (t >> 5)], 1u << (t & 31));
    }
  __syncthreads();
  int cnt = 0;
  if (tid < E)
    for (int w = 0; w < tw; ++w) {
      S.wpre[tid * tw + w] = (uint16_t)cnt;
      cnt += __popc(S.msk[tid * tw + w]);
    }
  const int ncg = (cnt + 16 * BCG - 1) / (16 * BCG);  // column groups
  // row blocks per column group: gate/up 64 rows (bf16, and the shared expert) or 128 rows
  // (mxfp4 routed experts); down 256 rows
  const int nrb_gu = a.I / 64, nrb_gr = a.xgm ? a.I / 128 : nrb_gu, nrb_dn = (H + 255) / 256;
  const int nrb_sh = a.Is / 64;  // the shared expert's gate/up items (bf16, 64 rows of Is)
  int4 tot;
  const int4 pre = block_excl_scan4(int4{cnt, cnt > 0 ? 1 : 0, ncg * nrb_gr, ncg * nrb_dn}, S.wsum, tid, tot);
  const int U = tot.y;
  int* ue = ut_arr(a, 0);
  int* uoff = ut_arr(a, 1);
  int* ucnt = ut_arr(a, 2);
  int* gpre = ut_arr(a, 3);
  int* dpre = ut_arr(a, 4);
  if (tid < E) S.eoff[tid] = pre.x;
  if (g == 0 && tid < E) {
    if (cnt > 0) {
      const int u = pre.y;
      ue[u] = tid; uoff[u] = pre.x; ucnt[u] = cnt; gpre[u] = pre.z; dpre[u] = pre.w;
    }
  }
  if (g == 0 && tid == 0) {  // the shared expert is slot U, over every token
    const int ncs = a.Is ? (T + 16 * BCG - 1) / (16 * BCG) : 0;
    ue[U] = -1; uoff[U] = n; ucnt[U] = a.Is ? T : 0; gpre[U] = tot.z; dpre[U] = tot.w;
    ue[U + 1] = -1; uoff[U + 1] = n + T; ucnt[U + 1] = 0;
    gpre[U + 1] = tot.z + ncs * nrb_sh;
    dpre[U + 1] = tot.w + ncs * nrb_dn;
    a.tab[0] = U; a.tab[1] = gpre[U + 1]; a.tab[2] = dpre[U + 1];
    if (a.out_n) a.out_n[0] = U;
  }
  __syncthreads();
  // this workgroup's pairs: experts e with e mod ng == g (the scattered stores spread over ng CUs)
#pragma unroll
  for (int m = 0; m < PPT; ++m) {
    const int i = tid + BPERM_NTH * m;
    const int t = pte[m] >> 16, e = pte[m] & 0xFFFF;
    if (i < n && e % ng == g) {
      const float wt = a.wts[i], rv = a.rinv[t];
      const int w = t >> 5;
      const int p = S.eoff[e] + S.wpre[e * tw + w] + __popc(S.msk[e * tw + w] & ((1u << (t & 31)) - 1u));
      a.blist[p] = t;
      a.bw[p] = wt;
      a.brv[p] = rv;
      a.bpos[i] = p;
    }
  }
  if (a.Is)
    for (int t = tid + BPERM_NTH * g; t < T; t += BPERM_NTH * ng) {
      a.blist[n + t] = t;
      a.bw[n + t] = 1.0f;
      a.brv[n + t] = a.rinv[t];
    }
}

// Geometry of one tick of the gathered expert kernels. bf16: one 128-wide window per tick, the
// B windows as 16 token rows of their 512-byte hi/lo fragment windows, rows BRS bytes apart;
// gate/up items are 64 rows, 4 row tiles x 2 K halves. mxfp4: two windows per tick (half the
// bytes of A per tick of bf16: two ticks of codes, scale bytes and gathered columns is what the
// registers hold), the B windows as MX-fp8 hi/lo operands with their scale words (MXW bytes per
// 16 columns); gate/up items are 128 rows, one row tile per wave over the whole reduction, so the
// gathered columns are half the share of an item's bytes they would be with K halves.
template <bool GU, bool MX>
struct BGeo {
  static constexpr int NKH = (GU && !MX) ? 2 : 1;           // K halves
  static constexpr int NWT = MX ? 2 : 1;                    // windows per tick
  static constexpr int RBR = GU ? (MX ? 128 : 64) : 256;    // rows per item (gate/up: of each matrix)
  static constexpr int DEPTH = BD;                          // ticks of loads in flight + 1
  static constexpr int NCB = NKH * NWT * BCG;               // 16-column B windows per tick
  static constexpr int CBB = MX ? MXW : 16 * 528;           // ring bytes per B window
  static constexpr int NCH = MX ? NCB * 256 / NTH : NCB;    // 16-byte B pieces per thread and tick
  static constexpr int RING = NCB * CBB;                    // ring bytes per slot
};
static_assert(BCG == 2, "the staging maps below assume two column tiles per item");
// bf16 ring rows: a token's 512-byte window plus 16 bytes, so the matrix-core lanes of 16
// columns (rows BRS apart, same piece) fall in different LDS banks
constexpr int BRS = 528;

// A operands of one tick for one wave: bf16, two 16-row bands x four k-steps of one window;
// mxfp4, two bands x two windows of codes (v[band * 2 + window]) and their scale bytes
struct BWin {
  u32x4 v[8];
  uint32_t sc[4];
};

// B pieces of one tick held by one thread (and, mxfp4, one scale word)
struct BReg {
  u32x4 v[4];
  uint32_t s;
};

// wave-uniform description of a gathered item for one wave
struct BItem {
  int u, off, cnt, col0;  // slot, list offset, tokens, first column (rank) of the item
  int rb;                 // row block
  bool shared;
  bool cached;            // the slot's weights are read by several column groups
  uint32_t aoff;          // byte offset of the wave's first A band (codes for mxfp4) in its tensor
  uint32_t soff;          // byte offset of its scales (mxfp4)
  int nwk;                // 128-wide windows of its rows' reduction (down: I, or Is for the shared expert)
  uint32_t band2;         // bf16 down: byte offset of its second row tile from the first
};

template <bool GU>
struct BSmem {
  static constexpr int RB = BGeo<GU, false>::RING > BGeo<GU, true>::RING ? BGeo<GU, false>::RING
                                                                          : BGeo<GU, true>::RING;
  alignas(16) uint8_t ring[2][RB];
  float red[GU ? 4 * 2 * BCG * 256 : 1];
  float act[GU ? 8 * BCG * 256 : 1];
  int ue[MAX_E + 2], uoff[MAX_E + 2], ucnt[MAX_E + 2], pre[MAX_E + 2];
};

template <bool GU, bool MX>
__device__ __forceinline__ BItem b_item(const BArgs& a, const BSmem<GU>& S, int U, int idx, int wave) {
  // slot: the largest u <= U with pre[u] <= idx (every slot below U + 1 with items has pre
  // strictly increasing)
  int lo = 0, hi = U;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (S.pre[mid] <= idx) lo = mid; else hi = mid - 1;
  }
  BItem d;
  d.u = lo;
  const int loc = idx - S.pre[lo];
  d.off = S.uoff[lo];
  d.cnt = S.ucnt[lo];
  // column groups fastest: the items that read the same weights are consecutive, so they run
  // together on one XCD (see the item order in bexp_run) and all but the first read hit its L2
  const int ncg = (d.cnt + 16 * BCG - 1) / (16 * BCG);
  const int cg = loc % ncg;
  d.rb = loc / ncg;
  d.col0 = cg * BCG * 16;
  d.cached = ncg > 1;
  const int e = S.ue[lo];
  d.shared = e < 0;
  const uint32_t eb = d.shared ? 0u : (uint32_t)e;
  // gate/up wave: rows rb RBR + 16 rt of gate and up, rt = w mod 4 (bf16, K half w / 4) or w
  // (mxfp4); down wave w: row tiles rb 256 + 32 w (+ 16)
  const uint32_t row = GU ? eb * (uint32_t)a.I + (uint32_t)(d.rb * BGeo<GU, MX>::RBR + 16 * (MX ? wave : (wave & 3)))
                          : eb * (uint32_t)a.H + (uint32_t)(d.rb * 256 + 32 * wave);
  const uint32_t K = GU ? (uint32_t)a.H : (uint32_t)(d.shared ? a.Is : a.I);  // reduction length of a row
  d.aoff = MX ? row * (K / 2) : row * (K * 2);
  d.soff = MX ? row * (K / 32) : 0u;
  if constexpr (!GU) {  // gate/up items all reduce over H
    d.nwk = (int)K / WIN;
    d.band2 = 16u * K * 2u;
  } else {
    d.nwk = a.H / WIN;
    d.band2 = 0u;
  }
  d.u = __builtin_amdgcn_readfirstlane(d.u);
  d.off = __builtin_amdgcn_readfirstlane(d.off);
  d.cnt = __builtin_amdgcn_readfirstlane(d.cnt);
  d.col0 = __builtin_amdgcn_readfirstlane(d.col0);
  d.rb = __builtin_amdgcn_readfirstlane(d.rb);
  d.aoff = __builtin_amdgcn_readfirstlane(d.aoff);
  d.soff = __builtin_amdgcn_readfirstlane(d.soff);
  d.cached = __builtin_amdgcn_readfirstlane((int)d.cached) != 0;
  d.shared = __builtin_amdgcn_readfirstlane((int)d.shared) != 0;
  if constexpr (!GU) {
    d.nwk = __builtin_amdgcn_readfirstlane(d.nwk);
    d.band2 = __builtin_amdgcn_readfirstlane(d.band2);
  }
  return d;
}

// One phase of a gathered expert kernel: items base .. base + n_items - 1 of one format, dealt
// m G + position, where a workgroup's position is its XCD-grouped slot (the 32 workgroups of an
// XCD take consecutive items, which share their gathered columns and repeated weights in that
// XCD's L2) rotated by rot, so a phase that follows another starts its deal after the
// workgroups the first one loaded.
// With rfull >= 0, only rounds 0 .. rfull - 1 go to every workgroup; the items after them are dealt
// over the workgroups at positions 0 .. nfree - 1 only (item rfull G + (m - rfull) nfree + position).
// kwin: windows of the down reduction of the phase's longest items (the layer's I, or Is when the
// phase holds shared items of a larger size); an item with a shorter reduction treats the windows
// past it as zero.
template <bool GU, bool MX>
__device__ void bexp_run(const BArgs& a, BSmem<GU>& S, int U, int base, int n_items, int rot, int tid,
                         int lane, int wave, int kwin, int rfull = -1, int nfree = 0) {
  using GE = BGeo<GU, MX>;
  const int G = gridDim.x, b = blockIdx.x;
  const int slotb = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  const int pos = (slotb - rot % G + G) % G;
  const bool split = rfull >= 0 && nfree > 0 && rfull * G <= n_items;
  const int rest = split ? n_items - rfull * G : 0;
  const int n_my = !split ? (pos < n_items ? (n_items - pos + G - 1) / G : 0)
                          : rfull + ((pos < nfree && pos < rest) ? (rest - pos + nfree - 1) / nfree : 0);
  if (n_my == 0) return;  // uniform over the workgroup
  auto gidx = [&](int m) {
    return (!split || m < rfull) ? m * G + pos : rfull * G + (m - rfull) * nfree + pos;
  };

  const int H = a.H, I = a.I;
  const int nwt = H / WIN;                     // windows of a token row (gate/up B source)
  const int nwk = GU ? nwt : kwin;             // windows of the A reduction (the phase's longest)
  const int nwh = GE::NKH == 2 ? (nwk + 1) / 2 : nwk;  // windows per K half
  const int ns = (nwh + GE::NWT - 1) / GE::NWT;        // ticks per item
  const int ticks = n_my * ns;
  const int kh = GE::NKH == 2 ? (wave >> 2) : 0;
  const uint32_t E = a.E;
  const uint32_t anum = GU ? E * (uint32_t)I * H : E * (uint32_t)H * I;  // values of a routed tensor
  const rsrc_t r0 = buf_rsrc(GU ? a.wg : a.wd, MX ? anum / 2 : anum * 2);
  const rsrc_t r1 = buf_rsrc(a.wu, GU ? (MX ? anum / 2 : anum * 2) : 0);
  const rsrc_t q0 = buf_rsrc(GU ? a.sg : a.sd, MX ? anum / 32 : 0);
  const rsrc_t q1 = buf_rsrc(a.su, (GU && MX) ? anum / 32 : 0);
  const uint32_t snum = (uint32_t)a.Is * H;  // values of a shared-expert tensor (bf16)
  const rsrc_t s0 = buf_rsrc(GU ? a.shg : a.shd, snum * 2), s1 = buf_rsrc(a.shu, GU ? snum * 2 : 0);
  const uint32_t vl = (uint32_t)lane * 16u;
  const int npos = a.T * a.K + a.T;
  const int nwa = max(I, a.Is) / WIN;  // windows per list position of the bf16 down operands
  const int bwr = GU ? nwt : (MX ? I / WIN : nwa);  // windows per B source row
  // items of one length (every gate/up item; down unless a shared expert of another size shares
  // the phase) keep the phase's window count, a loop invariant, in their window checks
  const bool mixed = !GU && !MX && a.Is != 0 && a.Is != I;
  const uint8_t* bsrc = MX ? (GU ? a.xgm : a.afm) : (GU ? a.xg : a.af);
  const rsrc_t rx = buf_rsrc(bsrc, (uint32_t)(GU ? a.T : npos + 16) * (uint32_t)bwr * (MX ? MXT : 512));
  // B staging. bf16: thread tid holds 16-byte piece tid % 32 of column tid / 32 for every (K
  // half, column tile): 32 threads copy one column's 512-byte window, contiguous in memory and
  // in its ring row. mxfp4: thread tid holds piece (tid / 16) % 16
  // of column tid % 16 of column tile (tid / 256) % 2 for the B windows (tid / 256) + 2 m, and,
  // below NCB 64, scale word tid % 4 of column (tid / 4) % 16 of B window tid / 64. Sixteen
  // consecutive lanes always write sixteen columns' pieces 32 bytes apart into the ring.
  const int bc = tid >> 5, bpc = tid & 31;
  const int mc = tid & 15, mch = (tid >> 4) & 15, mct = (tid >> 8) & 1;
  const int scb = tid >> 6, sc_c = (tid >> 2) & 15, sblk = tid & 3;

  auto item_of = [&](int m) {
    const int mm = m < n_my ? m : n_my - 1;  // past the end: the last item again (valid loads)
    return b_item<GU, MX>(a, S, U, base + gidx(mm), wave);
  };
  // window of B window-slot (K half h, tick window v) at tick step, and whether it exists
  auto win_of = [&](int h, int v, int step, bool& ok) {
    const int wl = step * GE::NWT + v;
    const int w = h * nwh + wl;
    ok = wl < nwh && w < nwk;
    return w;
  };
  auto load_a = [&](BWin& W, const BItem& d, int step) {
    if constexpr (!MX) {
      const int w = GU ? kh * ns + step : step;
      const uint32_t so = d.aoff + (uint32_t)w * 4096u;
      // a window past the item's reduction reads on into the tensor (finite values, or zeros past
      // its end) and meets zero B operands
      const rsrc_t ra = d.shared ? s0 : r0, rb2 = d.shared ? s1 : r1;
      // down: the second tile, 16 rows below (gate/up keeps the expression its schedule was tuned with)
      const uint32_t band2 = GU ? (uint32_t)(16 * I * 2) : d.band2;
      if (d.cached) {  // read again by the slot's other column groups: keep in L2
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          W.v[j] = bld16_cached(ra, vl + j * 1024, so);
          W.v[4 + j] = GU ? bld16_cached(rb2, vl + j * 1024, so) : bld16_cached(ra, vl + j * 1024, so + band2);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          W.v[j] = bld16(ra, vl + j * 1024, so);
          W.v[4 + j] = GU ? bld16(rb2, vl + j * 1024, so) : bld16(ra, vl + j * 1024, so + band2);
        }
      }
    } else {
      // band i: gate / up rows (gate/up), or row tile i (down); a window past the reduction
      // reads the half's first window (finite codes and scales, multiplied by zero B)
      const uint32_t c2 = GU ? 0u : (uint32_t)(16 * (I / 2)), s2 = GU ? 0u : (uint32_t)(16 * (I / 32));
#pragma unroll
      for (int v = 0; v < GE::NWT; ++v) {
        bool ok;
        int w = win_of(kh, v, step, ok);
        if (!ok) w = kh * nwh;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const rsrc_t rc = (GU && i) ? r1 : r0, rs = (GU && i) ? q1 : q0;
          const uint32_t co = d.aoff + (uint32_t)w * 1024u + (i ? c2 : 0u);
          const uint32_t sco = d.soff + (uint32_t)w * 64u + (i ? s2 : 0u);
          if (d.cached) {
            W.v[i * GE::NWT + v] = bld16_cached(rc, vl, co);
            W.sc[i * GE::NWT + v] = __builtin_amdgcn_raw_buffer_load_b8(rs, (uint32_t)lane, sco, 0);
          } else {
            W.v[i * GE::NWT + v] = bld16(rc, vl, co);
            W.sc[i * GE::NWT + v] = bld1(rs, (uint32_t)lane, sco);
          }
        }
      }
    }
  };
  // gathered B pieces of one tick; padding columns and missing windows read past the resource
  // (zeros, with no memory access: every real offset is far below 2^31)
  int ld_nwk = nwk;  // windows of the load cursor's item (read by down loads of mixed lengths)
  auto load_b = [&](BReg& R, const int (&src)[2], int step) {
    if constexpr (!MX) {
#pragma unroll
      for (int h = 0; h < GE::NKH; ++h) {
        bool okw;
        const int w = win_of(h, 0, step, okw);
        // down items shorter than the phase's longest (a shared expert of another size): their
        // windows past their own reduction take zero B operands
        if constexpr (!GU) okw = okw && (!mixed || w < ld_nwk);
#pragma unroll
        for (int ct = 0; ct < BCG; ++ct) {
          const bool ok = src[ct] >= 0 && okw;
          const uint32_t o = ok ? (uint32_t)((src[ct] * bwr + w) * 512 + bpc * 16) : 0x80000000u;
          R.v[h * BCG + ct] = __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < GE::NCH; ++m) {
        const int hv = ((tid >> 8) + 2 * m) >> 1;  // B window index / BCG
        bool okw;
        const int w = win_of(hv / GE::NWT, hv % GE::NWT, step, okw);
        const bool ok = src[0] >= 0 && okw;
        const uint32_t o = ok ? (uint32_t)((src[0] * bwr + w) * MXT + mch * 16) : 0x80000000u;
        R.v[m] = __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 0);
      }
      {
        const int hv = scb >> 1;
        bool okw;
        const int w = win_of(hv / GE::NWT, hv % GE::NWT, step, okw);
        const bool ok = tid < GE::NCB * 64 && src[1] >= 0 && okw;
        const uint32_t o = ok ? (uint32_t)((src[1] * bwr + w) * MXT + 256 + sblk * 4) : 0x80000000u;
        R.s = __builtin_amdgcn_raw_buffer_load_b32(rx, o, 0, 0);
      }
    }
  };
  auto store_b = [&](const BReg& R, int slot) {
    uint8_t* ring = S.ring[slot];
    if constexpr (!MX) {
#pragma unroll
      for (int h = 0; h < GE::NKH; ++h)
#pragma unroll
        for (int ct = 0; ct < BCG; ++ct)
          *reinterpret_cast<u32x4*>(ring + (h * BCG + ct) * GE::CBB + bc * BRS + bpc * 16) = R.v[h * BCG + ct];
    } else {
#pragma unroll
      for (int m = 0; m < GE::NCH; ++m) {
        const int cb = (tid >> 8) + 2 * m;
        const int part = mch >> 3, k8 = mch & 7;  // hi / lo, then (lane quad, 16-byte half)
        const int o = cb * MXW + part * 2048 + (mc + 16 * (k8 >> 1)) * 32 + 16 * (k8 & 1);
        *reinterpret_cast<u32x4*>(ring + o) = R.v[m];
      }
      if (tid < GE::NCB * 64)
        *reinterpret_cast<uint32_t*>(ring + scb * MXW + 4096 + (sc_c + 16 * sblk) * 4) = R.s;
    }
  };
  // the thread's B sources for an item: the token (gate/up) or list position (down) of each of
  // its columns, -1 past the item's tokens
  auto src_of = [&](const BItem& d, int (&src)[2]) {
    int r[2];
    if constexpr (!MX) {
      r[0] = d.col0 + bc;
      r[1] = d.col0 + 16 + bc;
    } else {
      r[0] = d.col0 + 16 * mct + mc;
      r[1] = d.col0 + 16 * (scb & 1) + sc_c;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int p = d.off + (r[k] < d.cnt ? r[k] : 0);
      src[k] = r[k] < d.cnt ? (GU ? a.blist[p] : p) : -1;
    }
  };

  // Cursors: the A and B loads of tick t + DEPTH - 1 are issued at tick t (B is stored into the
  // LDS ring at the end of tick t + DEPTH - 2), math at tick t. Vector memory results complete in issue
  // order, so every load whose result steers later loads (the column sources) is issued one
  // item ahead, and a wait for it never drains loads that were issued for later ticks.
  BWin W[GE::DEPTH];
  BReg R[GE::DEPTH];
  int ma = 0, sa = 0;  // load cursor (item, step)
  BItem da = item_of(0);
  if constexpr (!GU) ld_nwk = da.nwk;
  int srca[2], srcn[2];
  src_of(da, srca);
  src_of(item_of(1), srcn);
  auto advance = [&]() {
    if (++sa == ns) {
      sa = 0;
      ++ma;
      da = item_of(ma);
      if constexpr (!GU) ld_nwk = da.nwk;
      srca[0] = srcn[0];
      srca[1] = srcn[1];
      src_of(item_of(ma + 1), srcn);
    }
  };
#pragma unroll
  for (int j = 0; j < GE::DEPTH - 1; ++j) {
    load_a(W[j], da, sa);
    load_b(R[j], srca, sa);
    advance();
  }
  store_b(R[0], 0);
  __syncthreads();

  int mcur = 0, scur = 0;  // math cursor
  BItem dc = item_of(0);
  f32x4 acc[2][BCG];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int ct = 0; ct < BCG; ++ct) acc[i][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  // per-column epilogue factors of the math cursor's item (gate/up): RMSNorm factor and weight,
  // requested when the item's math starts and used at its last tick
  float crv[BCG], cw[BCG];
  auto col_factors = [&](const BItem& d) {
    if (!GU) return;
#pragma unroll
    for (int ct = 0; ct < BCG; ++ct) {
      const int r = d.col0 + 16 * ct + (lane & 15);
      const int p = d.off + (r < d.cnt ? r : 0);
      crv[ct] = a.brv[p];
      cw[ct] = a.bw[p];
    }
  };
  col_factors(dc);

  for (int t0 = 0;; t0 += GE::DEPTH) {
#pragma unroll
    for (int r = 0; r < GE::DEPTH; ++r) {
      const int t = t0 + r;
      const int ib = (r + GE::DEPTH - 1) % GE::DEPTH;  // buffers of tick t + DEPTH - 1
      load_a(W[ib], da, sa);
      load_b(R[ib], srca, sa);
      advance();
      __builtin_amdgcn_sched_barrier(0);
      // math of tick t
      {
        const uint8_t* ring = S.ring[t & 1];
#pragma unroll
        for (int ct = 0; ct < BCG; ++ct)
          if (ct == 0 || dc.col0 + 16 * ct < dc.cnt) {  // a column tile of padding only: skipped
            if constexpr (!MX) {
              // lane (column c, quad q) reads piece (2 j + hl) 4 + q of its column's row
              const uint8_t* rg = ring + (kh * BCG + ct) * GE::CBB + (lane & 15) * BRS + (lane >> 4) * 16;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const u32x4 bh = *reinterpret_cast<const u32x4*>(rg + (j * 2 + 0) * 64);
                const u32x4 bl = *reinterpret_cast<const u32x4*>(rg + (j * 2 + 1) * 64);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                  acc[i][ct] = mfma16(W[r].v[i * 4 + j], bh, acc[i][ct]);
                  acc[i][ct] = mfma16(W[r].v[i * 4 + j], bl, acc[i][ct]);
                }
              }
            } else {
#pragma unroll
              for (int v = 0; v < GE::NWT; ++v) {
                const uint8_t* cbp = ring + ((kh * GE::NWT + v) * BCG + ct) * MXW;
                const u32x4 bh0 = *reinterpret_cast<const u32x4*>(cbp + lane * 32);
                const u32x4 bh1 = *reinterpret_cast<const u32x4*>(cbp + lane * 32 + 16);
                const u32x4 bl0 = *reinterpret_cast<const u32x4*>(cbp + 2048 + lane * 32);
                const u32x4 bl1 = *reinterpret_cast<const u32x4*>(cbp + 2048 + lane * 32 + 16);
                const uint32_t bsc = *reinterpret_cast<const uint32_t*>(cbp + 4096 + lane * 4);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                  const int k = i * GE::NWT + v;
                  acc[i][ct] = mfma_mx(W[r].v[k], W[r].sc[k], bh0, bh1, bsc, 0, acc[i][ct]);
                  acc[i][ct] = mfma_mx(W[r].v[k], W[r].sc[k], bl0, bl1, bsc, 1, acc[i][ct]);
                }
              }
            }
          }
      }
      if (scur + 1 == ns) {  // the item's last tick: epilogue (uniform over the workgroup)
        if constexpr (GU && !MX) {
          const int rt = wave & 3;
          if (kh == 1)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int ct = 0; ct < BCG; ++ct)
                *reinterpret_cast<f32x4*>(&S.red[((rt * 2 + i) * BCG + ct) * 256 + lane * 4]) = acc[i][ct];
          __syncthreads();
          if (kh == 0) {
#pragma unroll
            for (int ct = 0; ct < BCG; ++ct) {
              const f32x4 g2 = *reinterpret_cast<const f32x4*>(&S.red[((rt * 2 + 0) * BCG + ct) * 256 + lane * 4]);
              const f32x4 u2 = *reinterpret_cast<const f32x4*>(&S.red[((rt * 2 + 1) * BCG + ct) * 256 + lane * 4]);
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const float g = (acc[0][ct][v] + g2[v]) * crv[ct];
                const float up = (acc[1][ct][v] + u2[v]) * crv[ct];
                // row 4 (lane / 16) + v, column lane % 16
                S.act[(rt * BCG + ct) * 256 + (4 * (lane >> 4) + v) * 16 + (lane & 15)] = silu(g) * up * cw[ct];
              }
            }
          }
          __syncthreads();
          if (tid < 4 * BCG * 2 * 16) {  // (rt, ct, half, column): 8 rows as down B operands
            const int c = tid & 15, half = (tid >> 4) & 1, ct = (tid >> 5) % BCG, rt2 = tid / (32 * BCG);
            const int rnk = dc.col0 + 16 * ct + c;
            if (rnk < dc.cnt) {
              uint32_t hi[8], lo[8];
#pragma unroll
              for (int i = 0; i < 8; ++i)
                split_bf16(S.act[(rt2 * BCG + ct) * 256 + (8 * half + i) * 16 + c], hi[i], lo[i]);
              u32x4 hv, lv;
              pack8(hi, hv);
              pack8(lo, lv);
              const int R0 = dc.rb * 64 + 16 * rt2 + 8 * half;  // intermediate row
              const int w = R0 / WIN, o = R0 % WIN, j = o / 32, qd = (o % 32) / 8;
              uint8_t* dst = a.af + ((size_t)(dc.off + rnk) * nwa + w) * 512;
              *reinterpret_cast<u32x4*>(dst + ((j * 2 + 0) * 4 + qd) * 16) = hv;
              *reinterpret_cast<u32x4*>(dst + ((j * 2 + 1) * 4 + qd) * 16) = lv;
            }
          }
        } else if constexpr (GU) {
          // mxfp4: each wave holds whole sums for its 16 rows; SwiGLU into the act tile, then
          // (ct, 32-row block bb, half h, column c): 16 rows quantised as MX-fp8 hi/lo, the block
          // maximum shared by the two halves (lanes c and c + 16 of one wave)
#pragma unroll
          for (int ct = 0; ct < BCG; ++ct)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float g = acc[0][ct][v] * crv[ct], up = acc[1][ct][v] * crv[ct];
              S.act[(wave * BCG + ct) * 256 + (4 * (lane >> 4) + v) * 16 + (lane & 15)] = silu(g) * up * cw[ct];
            }
          __syncthreads();
          if (tid < BCG * 4 * 2 * 16) {
            const int c = tid & 15, h = (tid >> 4) & 1, bb = (tid >> 5) & 3, ct = tid >> 7;
            float v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = S.act[((2 * bb + h) * BCG + ct) * 256 + j * 16 + c];
            uint32_t hi[4], lo[4];
            int eh, el;
            mx8_quant<16, true>(v, hi, lo, eh, el);
            const int rnk = dc.col0 + 16 * ct + c;
            if (rnk < dc.cnt) {
              const int R0 = dc.rb * 128 + 32 * bb;  // intermediate row of the block
              uint8_t* tw = a.afm + ((size_t)(dc.off + rnk) * (I / WIN) + R0 / WIN) * MXT;
              mx8_store16_tok(tw, (R0 % WIN) / 32, h, hi, lo, eh, el);
            }
          }
        } else {
          // lane: column lane % 16, rows 4 (lane / 16) .. + 3 of each of the wave's two tiles
#pragma unroll
          for (int ct = 0; ct < BCG; ++ct) {
            const int rnk = dc.col0 + 16 * ct + (lane & 15);
            if (rnk < dc.cnt) {
              float* dst = a.part + (size_t)(dc.off + rnk) * H;
#pragma unroll
              for (int i = 0; i < 2; ++i) {
                const int row = dc.rb * 256 + 32 * wave + 16 * i + 4 * (lane >> 4);
                if (row < H) *reinterpret_cast<f32x4*>(dst + row) = acc[i][ct];
              }
            }
          }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int ct = 0; ct < BCG; ++ct) acc[i][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        scur = 0;
        ++mcur;
        if (mcur < n_my) {
          dc = item_of(mcur);
          col_factors(dc);
        }
      } else {
        ++scur;
      }
      if (t + 1 == ticks) return;
      store_b(R[(r + 1) % GE::DEPTH], (t + 1) & 1);  // B of tick t + 1 (loads issued at tick t - 1)
      __syncthreads();
    }
  }
}

// The routed phase's deal in mxfp4 layers. With n1 < G shared items (bf16, one each on n1
// workgroups, which the routed deal's rotation puts last), a plain deal of the n2 routed items
// leaves those workgroups a whole shared item behind: at 512 tokens 128 of 256 workgroups took
// one shared item and four routed items and ended 22 us (gate/up) and 13 us (down) after the rest.
// So the routed rounds r0, r0 + 1, ... go only to the G - n1 workgroups without a shared item, r0
// chosen to minimise the larger of the two loads, a shared item counted as SC / 2 routed items
// (gate/up 3 / 2, down 5 / 2: the per-item times measured at 512 tokens). Returns (r0, G - n1), or
// (-1, 0) for the plain deal. The deal stays a bijection onto the items whatever the counts.
__device__ __forceinline__ int2 mx_tail_deal(int n2, int n1, int G, bool gu) {
  if (n1 <= 0 || n1 >= G || n2 < G) return int2{-1, 0};
  const int SC = gu ? 3 : 5, nf = G - n1;
  // loads in half routed items: shared workgroups SC + 2 r0; the others 2 (r0 + ceil((n2 - r0 G) / nf))
  auto load = [&](int x) {
    const int rest = n2 - x * G;
    return max(SC + 2 * x, 2 * (x + (rest + nf - 1) / nf));
  };
  const int plain = max(SC + 2 * ((n2 - nf + G - 1) / G), 2 * ((n2 + G - 1) / G));
  int best = 0, bl = load(0);
  for (int x = 1; x * G <= n2; ++x)  // the most full rounds among the lightest deals
    if (load(x) <= bl) { bl = load(x); best = x; }
  return bl < plain ? int2{best, nf} : int2{-1, 0};
}

// Gathered gate/up (GU) or down items. bf16 layers: one phase over every item. mxfp4 layers: the
// shared expert's items (bf16) first, then the routed experts' (mxfp4), in one launch.
template <bool GU, bool MXL>
__global__ void __launch_bounds__(NTH) k_bexp(BArgs a) {
  __shared__ BSmem<GU> S;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int U = __builtin_amdgcn_readfirstlane(a.tab[0]);
  for (int i = tid; i <= U + 1; i += NTH) {
    S.ue[i] = ut_arr(a, 0)[i];
    S.uoff[i] = ut_arr(a, 1)[i];
    S.ucnt[i] = ut_arr(a, 2)[i];
    S.pre[i] = ut_arr(a, GU ? 3 : 4)[i];
  }
  __syncthreads();
  const int routed = __builtin_amdgcn_readfirstlane(S.pre[U]);
  const int total = __builtin_amdgcn_readfirstlane(S.pre[U + 1]);
  if constexpr (!MXL) {
    bexp_run<GU, false>(a, S, U, 0, total, 0, tid, lane, wave, max(a.I, a.Is) / WIN);
  } else {
    const int n1 = total - routed;
    bexp_run<GU, false>(a, S, U, routed, n1, 0, tid, lane, wave, max(a.Is, WIN) / WIN);
    __syncthreads();  // the next phase reuses the LDS ring
    const int2 d = mx_tail_deal(routed, n1, gridDim.x, GU);
    bexp_run<GU, true>(a, S, U, 0, routed, n1, tid, lane, wave, a.I / WIN, d.x, d.y);
  }
}

// y[t][h] = sum_j P[pos(t, j)][h] + P[T K + t][h] (+ x[t][h]); one thread per four outputs
__global__ void __launch_bounds__(256) k_bcombine(BArgs a) {
  const int H = a.H, K = a.K, H4 = H / 4;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.T * H4) return;
  const int t = idx / H4, c = idx % H4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < K; ++j) {
    const float4 v = reinterpret_cast<const float4*>(a.part + (size_t)a.bpos[t * K + j] * H)[c];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  if (a.Is > 0) {
    const float4 v = reinterpret_cast<const float4*>(a.part + (size_t)(a.T * K + t) * H)[c];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  if (a.residual) {
    const float4 v = reinterpret_cast<const float4*>(a.x + (size_t)t * H)[c];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  reinterpret_cast<float4*>(a.y + (size_t)t * H)[c] = acc;
}

// ------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------
inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
  size_t ctr, xfrag, xfrag_sh, plog, psq, afrag, afrag_sh, part, total;
  int umax, hs;
};

int router_splits(int H) { return H >= 2048 ? HS_MAX : (H >= 1024 ? 2 : 1); }

Layout make_layout(const moe_layer* L, int k) {
  Layout o;
  const size_t H = L->hidden, E = L->n_experts, K = L->top_k, I = L->inter, Is = L->shared_inter;
  o.umax = (int)((E < (size_t)KMAX * K) ? E : (size_t)KMAX * K);
  o.hs = router_splits(L->hidden);
  size_t off = 0;
  o.ctr = off;       off = align256(off + (size_t)N_CTR * CTR_STRIDE * 4);
  o.xfrag = off;    off = align256(off + H * 64);
  o.xfrag_sh = off; off = align256(off + H * 64);
  o.plog = off;     off = align256(off + (size_t)o.hs * KMAX * E * 4);
  o.psq = off;      off = align256(off + (size_t)o.hs * KMAX * 4);
  o.afrag = off;    off = align256(off + (size_t)o.umax * I * 64);
  o.afrag_sh = off; off = align256(off + Is * 64);
  o.part = off;     off = align256(off + (size_t)k * (K + 1) * H * 4);
  o.total = off;
  return o;
}

// workspace of the gathered path for T tokens
struct BLayout {
  size_t tab, ut, logits, psq, rinv, xg, ids, wts, blist, bw, brv, bpos, af, part, xgm, afm, total;
};

BLayout make_blayout(const moe_layer* L, int T) {
  BLayout o;
  const size_t H = L->hidden, E = L->n_experts, K = L->top_k, I = L->inter;
  const size_t n = (size_t)T * K + T;  // list positions: routed pairs, then the shared expert
  size_t off = 0;
  o.tab = off;    off = align256(off + 16);
  o.ut = off;     off = align256(off + 5 * (E + 2) * 4);
  const size_t ns = H / gr_slice((int)H);  // router column slices
  o.logits = off; off = align256(off + ns * T * E * 4);
  o.psq = off;    off = align256(off + ns * T * 4);
  o.rinv = off;   off = align256(off + (size_t)T * 4);
  o.xg = off;     off = align256(off + (size_t)T * H * 4);
  o.ids = off;    off = align256(off + (size_t)T * K * 4);
  o.wts = off;    off = align256(off + (size_t)T * K * 4);
  o.blist = off;  off = align256(off + n * 4);
  o.bw = off;     off = align256(off + n * 4);
  o.brv = off;    off = align256(off + n * 4);
  o.bpos = off;   off = align256(off + (size_t)T * K * 4);
  o.af = off;     off = align256(off + (n + 16) * std::max(I, (size_t)L->shared_inter) * 4);
  o.part = off;   off = align256(off + n * H * 4);
  const bool mx = L->wdtype == MOE_W_MXFP4;  // MX-fp8 B windows of the routed experts
  o.xgm = off;    off = align256(off + (mx ? (size_t)T * (H / WIN) * MXT : 0));
  o.afm = off;    off = align256(off + (mx ? (n + 16) * (I / WIN) * MXT : 0));
  o.total = off;
  return o;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned8(const void* p) { return ((uintptr_t)p & 7u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + nb && pb < pa + na;
}

int check_layer(const moe_layer* L) {
  if (!L) return MOE_ERR_NULL;
  const int H = L->hidden, E = L->n_experts, K = L->top_k, I = L->inter, Is = L->shared_inter;
  if (H < 128 || H > 2048 || H % 128 || (H > 1024 && H % 256)) return MOE_ERR_SHAPE;
  if (E < 1 || E > MAX_E) return MOE_ERR_SHAPE;
  if (K < 1 || K > MAX_K || K > E) return MOE_ERR_SHAPE;
  if (I < 128 || I > 1024 || I % 128) return MOE_ERR_SHAPE;
  if (Is != 0 && (Is < 128 || Is > 1024 || Is % 128)) return MOE_ERR_SHAPE;
  if (L->wdtype != MOE_W_BF16 && L->wdtype != MOE_W_MXFP4) return MOE_ERR_DTYPE;
  if (L->layout != MOE_LAYOUT_TILED) return MOE_ERR_DTYPE;
  if (L->wdtype == MOE_W_MXFP4 && H % 256) return MOE_ERR_SHAPE;  // mxfp4 kernels take whole 256-row down blocks
  if (!L->router_w || !L->w_gate || !L->w_up || !L->w_down) return MOE_ERR_NULL;
  if (L->wdtype == MOE_W_MXFP4 && (!L->s_gate || !L->s_up || !L->s_down)) return MOE_ERR_DTYPE;
  if (Is && (!L->sh_gate || !L->sh_up || !L->sh_down)) return MOE_ERR_NULL;
  const void* ptrs[] = {L->router_w, L->w_gate, L->w_up, L->w_down, L->s_gate, L->s_up, L->s_down,
                        L->sh_gate, L->sh_up, L->sh_down};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_ALIGN;
  if (!(L->rms_eps >= 0.0f) || L->rms_eps > 3.0e38f) return MOE_ERR_ARG;
  return MOE_OK;
}

// The single-block kernels give each wave whole 128-column windows of the down reduction (I / 128
// must divide the eight waves) and lay the shared expert's items out like the routed ones (Is = I).
// Layers outside that set take the gathered path for every k, which handles any multiple of 128.
bool block_shape_ok(const moe_layer* L) {
  const int I = L->inter, Is = L->shared_inter;
  return (I == 128 || I == 256 || I == 512 || I == 1024) && (Is == 0 || Is == I);
}
bool use_gather(const moe_layer* L, int k, uint32_t flags) {
  return k > KMAX || (flags & MOE_GATHER) || !block_shape_ok(L);
}

// A HIP error left pending by the caller's earlier work would be reported (and cleared) by the
// launch check of this call as if it were this call's; such a call enqueues nothing, returns
// MOE_ERR_HIP and leaves the error pending for the caller to read.
bool error_pending() { return hipPeekAtLastError() != hipSuccess; }

// A 64-bit value unique to each call in this process (a Weyl sequence from a random start), never
// zero: the tag of that call's completion flags, so flags left in a workspace by earlier calls, or
// any other stale contents, are not taken for this call's.
uint64_t next_epoch() {
  static const uint64_t base = [] {
    std::random_device rd;
    return ((uint64_t)rd() << 32) ^ (uint64_t)rd() ^ (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
  }();
  static std::atomic<uint64_t> n{0};
  uint64_t e;
  do {
    e = base + 0x9E3779B97F4A7C15ull * (n.fetch_add(1, std::memory_order_relaxed) + 1);
  } while (e == 0);
  return e;
}

// The current device's compute-unit count, looked up once per device (calls from several host
// threads may look it up together; they store the same value).
int num_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Records events[i] (any may be NULL) on the stream; false if a record fails.
bool mark(void* const* events, int i, hipStream_t s) {
  return !events || !events[i] || hipEventRecord((hipEvent_t)events[i], s) == hipSuccess;
}

// Workgroups of the expert kernels: one per CU; never fewer than shared-expert items (one each),
// nor than combine slices of the one-launch kernel (128 output float4s each).
int layer_grid(const Args& a) {
  return std::max(std::max(num_cus(), (a.k * a.H / 4 + 127) / 128), std::max(a.Is / 16, a.H / 64));
}

template <int WPW, int NWIN, bool MX>
bool launch_layer(const Args& a, hipStream_t s, void* const* ev) {
  const int cus = layer_grid(a);
  if (!mark(ev, 0, s)) return false;
  k_router<MX><<<a.ntile_e * a.hs, NTH, 0, s>>>(a);
  if (!mark(ev, 1, s)) return false;
  k_layer<WPW, NWIN, MX><<<cus, NTH, 0, s>>>(a);
  return mark(ev, 2, s) && mark(ev, 3, s) && mark(ev, 4, s);
}

template <int WPW, bool MX>
bool launch_nwin(const Args& a, hipStream_t s, void* const* ev) {
  switch (a.I / WIN) {
    case 1: return launch_layer<WPW, 1, MX>(a, s, ev);
    case 2: return launch_layer<WPW, 2, MX>(a, s, ev);
    case 4: return launch_layer<WPW, 4, MX>(a, s, ev);
    default: return launch_layer<WPW, 8, MX>(a, s, ev);
  }
}

// Scratch of moe_verify_block_noalloc: the workspace lives in this file-scope device array (one
// copy per GPU, held until the process ends) instead of a caller buffer. In host code `scratch`
// names a host-side stand-in, never the device copy: its device address is looked up once per
// device with hipGetSymbolAddress and only that address is passed to kernels.
__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES] = {};

// The current device's scratch address (looked up on the first call per device), or NULL with
// *status set to MOE_ERR_HIP.
void* device_scratch(int* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
    *status = MOE_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> g(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *status = MOE_ERR_HIP;
      return nullptr;
    }
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is outside the supported range";
    case MOE_ERR_DTYPE: return "unknown weight format or layout, or missing mxfp4 scales";
    case MOE_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_ALIAS: return "an output overlaps an input";
    case MOE_ERR_HIP: return "kernel launch failed";
    case MOE_ERR_ARG: return "bad flag bits or scalar argument";
    default: return "unknown status";
  }
}

size_t moe_verify_workspace_size(const moe_layer* layer, int32_t k_max) {
  if (check_layer(layer) != MOE_OK || k_max < 1 || k_max > BT_MAX) return 0;
  if (!block_shape_ok(layer)) return make_blayout(layer, k_max).total;
  const size_t small = make_layout(layer, std::min(k_max, (int32_t)KMAX)).total;
  return std::max(small, make_blayout(layer, k_max).total);
}

// the gathered path (k > 16 tokens, MOE_GATHER, or a layer outside the single-block shapes)
static int gather_impl(const moe_layer* L, const float* x, int32_t T, uint32_t flags, float* y,
                       int32_t* topk_ids, float* topk_w, int32_t* n_woken, void* workspace, size_t ws_bytes,
                       void* hip_stream, void* const* events) {
  const bool mx = L->wdtype == MOE_W_MXFP4;
  if (!aligned16(x) || !aligned16(y) || !aligned16(workspace) || (topk_ids && !aligned16(topk_ids)) ||
      (topk_w && !aligned16(topk_w)) || (n_woken && !aligned16(n_woken)))
    return MOE_ERR_ALIGN;
  const BLayout lay = make_blayout(L, T);
  if (ws_bytes < lay.total) return MOE_ERR_WORKSPACE;
  const size_t xy_bytes = (size_t)T * L->hidden * 4;
  const size_t ids_bytes = (size_t)T * L->top_k * 4;
  if (overlaps(x, xy_bytes, y, xy_bytes) || overlaps(y, xy_bytes, workspace, lay.total)) return MOE_ERR_ALIAS;
  if (overlaps(x, xy_bytes, workspace, lay.total)) return MOE_ERR_ALIAS;
  if (topk_ids && (overlaps(topk_ids, ids_bytes, workspace, lay.total) || overlaps(topk_ids, ids_bytes, y, xy_bytes)))
    return MOE_ERR_ALIAS;
  if (topk_w && (overlaps(topk_w, ids_bytes, workspace, lay.total) || overlaps(topk_w, ids_bytes, y, xy_bytes)))
    return MOE_ERR_ALIAS;
  if (n_woken && (overlaps(n_woken, 4, workspace, lay.total) || overlaps(n_woken, 4, y, xy_bytes)))
    return MOE_ERR_ALIAS;

  uint8_t* ws = (uint8_t*)workspace;
  BArgs a;
  a.x = x; a.y = y; a.out_ids = topk_ids; a.out_w = topk_w; a.out_n = n_woken;
  a.wr = L->router_w;
  a.wg = (const uint8_t*)L->w_gate; a.wu = (const uint8_t*)L->w_up; a.wd = (const uint8_t*)L->w_down;
  a.shg = (const uint8_t*)L->sh_gate; a.shu = (const uint8_t*)L->sh_up; a.shd = (const uint8_t*)L->sh_down;
  a.logits = (float*)(ws + lay.logits); a.psq = (float*)(ws + lay.psq); a.rinv = (float*)(ws + lay.rinv);
  a.xg = ws + lay.xg;
  a.ids = (int32_t*)(ws + lay.ids); a.wts = (float*)(ws + lay.wts); a.tab = (int32_t*)(ws + lay.tab);
  a.ut = (int32_t*)(ws + lay.ut); a.blist = (int32_t*)(ws + lay.blist); a.bw = (float*)(ws + lay.bw);
  a.brv = (float*)(ws + lay.brv); a.bpos = (int32_t*)(ws + lay.bpos); a.af = ws + lay.af;
  a.part = (float*)(ws + lay.part);
  a.sg = L->s_gate; a.su = L->s_up; a.sd = L->s_down;
  a.xgm = mx ? ws + lay.xgm : nullptr;
  a.afm = mx ? ws + lay.afm : nullptr;
  a.H = L->hidden; a.E = L->n_experts; a.K = L->top_k; a.I = L->inter; a.Is = L->shared_inter; a.T = T;
  a.pre_norm = (flags & MOE_PRE_RMSNORM) ? 1 : 0; a.residual = (flags & MOE_RESIDUAL) ? 1 : 0;
  a.eps = L->rms_eps;

  hipStream_t s = (hipStream_t)hip_stream;
  if (error_pending()) return MOE_ERR_HIP;  // the caller's own error stays pending
  const int cus = num_cus();
  const int n_rt = ((T + GR_T - 1) / GR_T) * ((a.E + GR_E - 1) / GR_E) * (a.H / gr_slice(a.H));
  bool ok = mark(events, 0, s);
  if (ok) {
    if (gr_slice(a.H) == 256) k_brouter<4><<<n_rt, BR_NTH, 0, s>>>(a);
    else                      k_brouter<2><<<n_rt, BR_NTH, 0, s>>>(a);
    k_btopk<<<(T + NW - 1) / NW, NTH, 0, s>>>(a);
    k_bperm<<<BPERM_G, BPERM_NTH, 0, s>>>(a);
    ok = mark(events, 1, s);
  }
  if (ok) {
    if (mx) k_bexp<true, true><<<cus, NTH, 0, s>>>(a);
    else    k_bexp<true, false><<<cus, NTH, 0, s>>>(a);
    ok = mark(events, 2, s);
  }
  if (ok) {
    if (mx) k_bexp<false, true><<<cus, NTH, 0, s>>>(a);
    else    k_bexp<false, false><<<cus, NTH, 0, s>>>(a);
    ok = mark(events, 3, s);
  }
  if (ok) {
    k_bcombine<<<(T * a.H / 4 + 255) / 256, 256, 0, s>>>(a);
    ok = mark(events, 4, s);
  }
  return (ok && hipGetLastError() == hipSuccess) ? MOE_OK : MOE_ERR_HIP;
}

// The single-block path's kernel arguments for one layer call on workspace ws (layout lay).
static Args block_args(const moe_layer* L, const float* x, int32_t k, uint32_t flags, float* y, int32_t* topk_ids,
                       float* topk_w, int32_t* n_woken, uint8_t* ws, const Layout& lay) {
  Args a;
  a.x = x; a.y = y; a.out_ids = topk_ids; a.out_w = topk_w; a.out_n = n_woken;
  a.wr = L->router_w;
  a.wg = (const uint8_t*)L->w_gate; a.wu = (const uint8_t*)L->w_up; a.wd = (const uint8_t*)L->w_down;
  a.sg = L->s_gate; a.su = L->s_up; a.sd = L->s_down;
  a.shg = (const uint8_t*)L->sh_gate; a.shu = (const uint8_t*)L->sh_up; a.shd = (const uint8_t*)L->sh_down;
  a.ctr = (uint32_t*)(ws + lay.ctr);
  a.xfrag = (u32x4*)(ws + lay.xfrag); a.xfrag_sh = (u32x4*)(ws + lay.xfrag_sh); a.plog = (float*)(ws + lay.plog); a.psq = (float*)(ws + lay.psq);
  a.afrag = (u32x4*)(ws + lay.afrag); a.afrag_sh = (u32x4*)(ws + lay.afrag_sh); a.part = (float*)(ws + lay.part);
  a.H = L->hidden; a.E = L->n_experts; a.K = L->top_k; a.I = L->inter; a.Is = L->shared_inter; a.k = k;
  a.hs = lay.hs; a.ntile_e = (L->n_experts + 15) / 16; a.umax = lay.umax;
  a.pre_norm = (flags & MOE_PRE_RMSNORM) ? 1 : 0; a.residual = (flags & MOE_RESIDUAL) ? 1 : 0;
  a.eps = L->rms_eps;
  return a;
}

static int verify_block_impl(const moe_layer* L, const float* x, int32_t k, uint32_t flags, float* y,
                             int32_t* topk_ids, float* topk_w, int32_t* n_woken, void* workspace,
                             size_t ws_bytes, void* hip_stream, void* const* events) {
  int st = check_layer(L);
  if (st != MOE_OK) return st;
  if (!x || !y || !workspace) return MOE_ERR_NULL;
  if (k < 1 || k > BT_MAX) return MOE_ERR_SHAPE;
  if (flags & ~(uint32_t)(MOE_PRE_RMSNORM | MOE_RESIDUAL | MOE_GATHER)) return MOE_ERR_ARG;
  if (use_gather(L, k, flags))
    return gather_impl(L, x, k, flags, y, topk_ids, topk_w, n_woken, workspace, ws_bytes, hip_stream, events);
  if (!aligned16(x) || !aligned16(y) || !aligned16(workspace) || (topk_ids && !aligned16(topk_ids)) ||
      (topk_w && !aligned16(topk_w)) || (n_woken && !aligned16(n_woken)))
    return MOE_ERR_ALIGN;
  const Layout lay = make_layout(L, k);
  if (ws_bytes < lay.total) return MOE_ERR_WORKSPACE;
  const size_t xy_bytes = (size_t)k * L->hidden * 4;
  const size_t ids_bytes = (size_t)k * L->top_k * 4;
  if (overlaps(x, xy_bytes, y, xy_bytes) || overlaps(y, xy_bytes, workspace, lay.total)) return MOE_ERR_ALIAS;
  if (overlaps(x, xy_bytes, workspace, lay.total)) return MOE_ERR_ALIAS;
  if (topk_ids && (overlaps(topk_ids, ids_bytes, workspace, lay.total) || overlaps(topk_ids, ids_bytes, y, xy_bytes)))
    return MOE_ERR_ALIAS;
  if (topk_w && (overlaps(topk_w, ids_bytes, workspace, lay.total) || overlaps(topk_w, ids_bytes, y, xy_bytes)))
    return MOE_ERR_ALIAS;
  if (n_woken && (overlaps(n_woken, 4, workspace, lay.total) || overlaps(n_woken, 4, y, xy_bytes)))
    return MOE_ERR_ALIAS;

  const Args a = block_args(L, x, k, flags, y, topk_ids, topk_w, n_woken, (uint8_t*)workspace, lay);

  hipStream_t s = (hipStream_t)hip_stream;
  if (error_pending()) return MOE_ERR_HIP;  // the caller's own error stays pending
  // the one-launch layer kernel's phases wait for each other: every workgroup must be resident
  if (layer_grid(a) > num_cus()) return MOE_ERR_SHAPE;
  const bool mx = L->wdtype == MOE_W_MXFP4;
  bool ok;
  if (L->hidden > 1024) ok = mx ? launch_nwin<2, true>(a, s, events) : launch_nwin<2, false>(a, s, events);
  else                  ok = mx ? launch_nwin<1, true>(a, s, events) : launch_nwin<1, false>(a, s, events);
  return (ok && hipGetLastError() == hipSuccess) ? MOE_OK : MOE_ERR_HIP;
}

int moe_verify_block(const moe_layer* L, const float* x, int32_t k, uint32_t flags, float* y,
                     int32_t* topk_ids, float* topk_w, int32_t* n_woken, void* workspace,
                     size_t ws_bytes, void* hip_stream) {
  return verify_block_impl(L, x, k, flags, y, topk_ids, topk_w, n_woken, workspace, ws_bytes, hip_stream,
                           nullptr);
}

int moe_verify_block_timed(const moe_layer* L, const float* x, int32_t k, uint32_t flags, float* y,
                           int32_t* topk_ids, float* topk_w, int32_t* n_woken, void* workspace,
                           size_t ws_bytes, void* hip_stream, void* const* events) {
  return verify_block_impl(L, x, k, flags, y, topk_ids, topk_w, n_woken, workspace, ws_bytes, hip_stream,
                           events);
}

int moe_verify_block_noalloc(const moe_layer* L, const float* x, int32_t k, uint32_t flags, float* y,
                             int32_t* topk_ids, float* topk_w, int32_t* n_woken, void* hip_stream) {
  const int st = check_layer(L);
  if (st != MOE_OK) return st;
  if (!x || !y) return MOE_ERR_NULL;
  if (k < 1 || k > BT_MAX) return MOE_ERR_SHAPE;
  if (flags & ~(uint32_t)(MOE_PRE_RMSNORM | MOE_RESIDUAL | MOE_GATHER)) return MOE_ERR_ARG;
  const size_t need = use_gather(L, k, flags) ? make_blayout(L, k).total : make_layout(L, k).total;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  if (error_pending()) return MOE_ERR_HIP;  // the caller's own error stays pending
  int lookup = MOE_OK;
  void* ws = device_scratch(&lookup);
  if (!ws) return lookup;
  return verify_block_impl(L, x, k, flags, y, topk_ids, topk_w, n_woken, ws, MOE_NOALLOC_SCRATCH_BYTES, hip_stream,
                           nullptr);
}

// Stack workspace: the single-block layout, then two ping-pong activation buffers.
struct StackLayout {
  Layout base;
  size_t pp0, pp1, total;
};
static StackLayout make_stack_layout(const moe_layer* L, int k) {
  StackLayout o;
  o.base = make_layout(L, k);
  size_t off = o.base.total;
  o.pp0 = off; off = align256(off + (size_t)k * L->hidden * 4);
  o.pp1 = off; off = align256(off + (size_t)k * L->hidden * 4);
  o.total = off;
  return o;
}
static bool same_shape(const moe_layer* a, const moe_layer* b) {
  return a->hidden == b->hidden && a->n_experts == b->n_experts && a->top_k == b->top_k && a->inter == b->inter &&
         a->shared_inter == b->shared_inter && a->wdtype == b->wdtype && a->layout == b->layout;
}

size_t moe_verify_stack_workspace_size(const moe_layer* layer, int32_t k_max) {
  if (check_layer(layer) != MOE_OK || k_max < 1 || k_max > KMAX || !block_shape_ok(layer)) return 0;
  return make_stack_layout(layer, k_max).total;
}

int moe_verify_stack(const moe_layer* layers, int32_t n_layers, const float* x, int32_t k, uint32_t flags, float* y,
                     int32_t* n_woken, void* workspace, size_t ws_bytes, void* hip_stream) {
  if (!layers || !x || !y || !workspace) return MOE_ERR_NULL;
  if (n_layers < 1 || n_layers > MOE_STACK_MAX_LAYERS) return MOE_ERR_SHAPE;
  for (int l = 0; l < n_layers; ++l) {
    const int st = check_layer(&layers[l]);
    if (st != MOE_OK) return st;
    if (!same_shape(&layers[0], &layers[l])) return MOE_ERR_SHAPE;
  }
  if (flags & ~(uint32_t)(MOE_PRE_RMSNORM | MOE_RESIDUAL)) return MOE_ERR_ARG;
  if (k < 1 || k > KMAX || !block_shape_ok(&layers[0])) return MOE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(y) || !aligned16(workspace) || (n_woken && !aligned16(n_woken)))
    return MOE_ERR_ALIGN;
  const StackLayout lay = make_stack_layout(&layers[0], k);
  if (ws_bytes < lay.total) return MOE_ERR_WORKSPACE;
  const size_t xy_bytes = (size_t)k * layers[0].hidden * 4, nw_bytes = (size_t)n_layers * 4;
  if (overlaps(x, xy_bytes, y, xy_bytes) || overlaps(x, xy_bytes, workspace, lay.total) ||
      overlaps(y, xy_bytes, workspace, lay.total))
    return MOE_ERR_ALIAS;
  if (n_woken && (overlaps(n_woken, nw_bytes, workspace, lay.total) || overlaps(n_woken, nw_bytes, y, xy_bytes) ||
                  overlaps(n_woken, nw_bytes, x, xy_bytes)))
    return MOE_ERR_ALIAS;
  hipStream_t s = (hipStream_t)hip_stream;
  if (error_pending()) return MOE_ERR_HIP;  // the caller's own error stays pending
  uint8_t* ws = (uint8_t*)workspace;
  float* pp[2] = {(float*)(ws + lay.pp0), (float*)(ws + lay.pp1)};
  const bool mx = layers[0].wdtype == MOE_W_MXFP4;
  for (int l = 0; l < n_layers; ++l) {
    const float* in = l == 0 ? x : pp[(l - 1) & 1];
    float* out = l == n_layers - 1 ? y : pp[l & 1];
    const Args a = block_args(&layers[l], in, k, flags, out, nullptr, nullptr, n_woken ? n_woken + l : nullptr, ws,
                              lay.base);
    if (layer_grid(a) > num_cus()) return MOE_ERR_SHAPE;  // every workgroup resident (see moe_verify_block)
    bool ok;
    if (layers[0].hidden > 1024) ok = mx ? launch_nwin<2, true>(a, s, nullptr) : launch_nwin<2, false>(a, s, nullptr);
    else                         ok = mx ? launch_nwin<1, true>(a, s, nullptr) : launch_nwin<1, false>(a, s, nullptr);
    if (!ok) return MOE_ERR_HIP;
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_pack_weights(int32_t wdtype, int32_t n_mats, int32_t rows, int32_t cols, const void* src,
                     const uint8_t* src_scales, void* dst, uint8_t* dst_scales, void* hip_stream) {
  if (!src || !dst) return MOE_ERR_NULL;
  if (wdtype != MOE_W_BF16 && wdtype != MOE_W_MXFP4) return MOE_ERR_DTYPE;
  if (wdtype == MOE_W_MXFP4 && (!src_scales || !dst_scales)) return MOE_ERR_NULL;
  if (n_mats < 1 || rows < 16 || rows % 16 || cols < 128 || cols % 128 || rows > (1 << 20) ||
      cols > (1 << 20) || n_mats > (1 << 20))
    return MOE_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(dst)) return MOE_ERR_ALIGN;
  const uint64_t elems = (uint64_t)n_mats * rows * cols;
  const size_t bytes = wdtype == MOE_W_BF16 ? elems * 2 : elems / 2;
  if (overlaps(src, bytes, dst, bytes)) return MOE_ERR_ALIAS;
  if (wdtype == MOE_W_MXFP4 && (overlaps(src_scales, elems / 32, dst_scales, elems / 32) ||
                                overlaps(dst_scales, elems / 32, src, bytes) ||
                                overlaps(dst_scales, elems / 32, dst, bytes) ||
                                overlaps(dst, bytes, src_scales, elems / 32)))
    return MOE_ERR_ALIAS;
  hipStream_t s = (hipStream_t)hip_stream;
  if (error_pending()) return MOE_ERR_HIP;  // the caller's own error stays pending
  const int grid = 2048;
  if (wdtype == MOE_W_BF16)
    k_pack_bf16<<<grid, 256, 0, s>>>((const uint8_t*)src, (uint8_t*)dst, rows, cols, elems / 8);
  else
    k_pack_mx<<<grid, 256, 0, s>>>((const uint8_t*)src, src_scales, (uint8_t*)dst, dst_scales, rows, cols,
                                   elems / 32);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// workspace of the acceptance: one 16-byte record (max, index, tag) per row and chunk
// records [rows][nchunks] of 16 bytes, then a generation word per sequence
size_t accept_rec_bytes(size_t rows, size_t nchunks) { return align256(rows * nchunks * 16); }
size_t accept_ws_bytes(size_t rows, size_t nchunks, size_t nseq) {
  return accept_rec_bytes(rows, nchunks) + align256(nseq * 4);
}

size_t accept_prefix_workspace_size(int32_t n_target, int32_t vocab) {
  if (n_target < 1 || n_target > 64 || vocab < 1 || vocab > (1 << 24)) return 0;
  const size_t nchunks = ((size_t)vocab + AM_CHUNK - 1) / AM_CHUNK;
  return accept_ws_bytes((size_t)n_target, nchunks, 1);
}

size_t accept_prefix_batch_workspace_size(int32_t n_seq, int32_t n_target, int32_t vocab) {
  if (n_seq < 1 || n_seq > 1024 || n_target < 1 || n_target > 64 || n_seq * n_target > 65535 || vocab < 1 ||
      vocab > (1 << 24))
    return 0;
  const size_t nchunks = ((size_t)vocab + AM_CHUNK - 1) / AM_CHUNK;
  return accept_ws_bytes((size_t)n_seq * n_target, nchunks, (size_t)n_seq);
}

int accept_prefix_batch(const float* logits, int32_t n_seq, int32_t n_target, int32_t vocab,
                        const int32_t* draft_ids, int32_t n_draft_max, const int32_t* n_draft,
                        int32_t* target_ids, int32_t* accepted, void* workspace, size_t ws_bytes,
                        void* hip_stream) {
  if (!logits || !target_ids || !accepted || !workspace || (n_draft_max > 0 && !draft_ids)) return MOE_ERR_NULL;
  if (n_seq < 1 || n_seq > 1024 || n_target < 1 || n_target > 64 || n_seq * n_target > 65535 || vocab < 1 ||
      vocab > (1 << 24) || n_draft_max < 0 || n_draft_max > n_target)
    return MOE_ERR_SHAPE;
  if (!aligned16(logits) || !aligned16(target_ids) || !aligned16(accepted) || !aligned16(workspace) ||
      (draft_ids && !aligned16(draft_ids)) || (n_draft && !aligned16(n_draft)))
    return MOE_ERR_ALIGN;
  const size_t need = accept_prefix_batch_workspace_size(n_seq, n_target, vocab);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  const size_t lbytes = (size_t)n_seq * n_target * vocab * 4;
  const size_t tbytes = (size_t)n_seq * n_target * 4, abytes = (size_t)n_seq * 4;
  if (overlaps(target_ids, tbytes, logits, lbytes) || overlaps(accepted, abytes, logits, lbytes) ||
      overlaps(target_ids, tbytes, workspace, need) || overlaps(accepted, abytes, workspace, need) ||
      overlaps(accepted, abytes, target_ids, tbytes))
    return MOE_ERR_ALIAS;
  const int nchunks = (vocab + AM_CHUNK - 1) / AM_CHUNK;
  hipStream_t s = (hipStream_t)hip_stream;
  if (error_pending()) return MOE_ERR_HIP;  // the caller's own error stays pending
  uint32_t* gen = (uint32_t*)((uint8_t*)workspace + accept_rec_bytes((size_t)n_seq * n_target, nchunks));
  k_accept<<<dim3(nchunks, n_seq * n_target), 256, 0, s>>>(logits, vocab, nchunks, n_target,
                                                           n_draft_max > 0 ? draft_ids : nullptr, n_draft_max, n_draft,
                                                           target_ids, accepted, (u32x4*)workspace, gen, next_epoch());
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int accept_prefix(const float* logits, int32_t n_target, int32_t vocab, const int32_t* draft_ids,
                  int32_t n_draft, int32_t* target_ids, int32_t* accepted, void* workspace,
                  size_t ws_bytes, void* hip_stream) {
  if (!logits || !target_ids || !accepted || !workspace || (n_draft > 0 && !draft_ids)) return MOE_ERR_NULL;
  if (n_target < 1 || n_target > 64 || vocab < 1 || vocab > (1 << 24) || n_draft < 0 || n_draft > n_target)
    return MOE_ERR_SHAPE;
  if (!aligned16(logits) || !aligned16(target_ids) || !aligned16(accepted) || !aligned16(workspace) ||
      (draft_ids && !aligned16(draft_ids)))
    return MOE_ERR_ALIGN;
  const size_t need = accept_prefix_workspace_size(n_target, vocab);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  const size_t lbytes = (size_t)n_target * vocab * 4;
  if (overlaps(target_ids, (size_t)n_target * 4, logits, lbytes) || overlaps(accepted, 4, logits, lbytes) ||
      overlaps(target_ids, (size_t)n_target * 4, workspace, need) || overlaps(accepted, 4, workspace, need) ||
      overlaps(accepted, 4, target_ids, (size_t)n_target * 4))
    return MOE_ERR_ALIAS;
  const int nchunks = (vocab + AM_CHUNK - 1) / AM_CHUNK;
  hipStream_t s = (hipStream_t)hip_stream;
  if (error_pending()) return MOE_ERR_HIP;  // the caller's own error stays pending
  uint32_t* gen = (uint32_t*)((uint8_t*)workspace + accept_rec_bytes((size_t)n_target, nchunks));
  k_accept<<<dim3(nchunks, n_target), 256, 0, s>>>(logits, vocab, nchunks, n_target, n_draft > 0 ? draft_ids : nullptr,
                                                   n_draft, nullptr, target_ids, accepted, (u32x4*)workspace, gen,
                                                   next_epoch());
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

constexpr int HEAD_GMAX = 1024;  // largest grid the head workspace provides for

// workspace: partial maxima pv [n][G] fp32, their rows pi [n][G], then the claim pool counters
size_t lm_head_accept_workspace_size(int32_t n_target, int32_t hidden, int32_t vocab) {
  if (n_target < 1 || n_target > KMAX || hidden < 1 || vocab < 1) return 0;
  return 2 * align256((size_t)n_target * HEAD_GMAX * 4) + (size_t)NGRP * HEAD_CTR_STRIDE * 8;
}

int lm_head_accept(const float* h, int32_t n_target, int32_t hidden, const void* w_head, int32_t vocab,
                   int32_t layout, const int32_t* draft_ids, int32_t n_draft, int32_t* target_ids,
                   int32_t* accepted, void* workspace, size_t ws_bytes, void* hip_stream) {
  if (!h || !w_head || !target_ids || !accepted || !workspace || (n_draft > 0 && !draft_ids)) return MOE_ERR_NULL;
  if (n_target < 1 || n_target > KMAX || n_draft < 0 || n_draft > n_target || hidden < WIN ||
      hidden > 2 * NW * WIN || hidden % WIN != 0 || vocab < 1)
    return MOE_ERR_SHAPE;
  const uint64_t v16 = ((uint64_t)vocab + 15) / 16 * 16;
  if (v16 * (uint64_t)hidden * 2 > 0xFFFFFFFFull) return MOE_ERR_SHAPE;  // 32-bit buffer offsets
  if (layout != MOE_LAYOUT_TILED) return MOE_ERR_DTYPE;
  if (!aligned16(h) || !aligned16(w_head) || !aligned16(target_ids) || !aligned16(accepted) ||
      !aligned16(workspace) || (draft_ids && !aligned16(draft_ids)))
    return MOE_ERR_ALIGN;
  const size_t need = lm_head_accept_workspace_size(n_target, hidden, vocab);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  const size_t hbytes = (size_t)n_target * hidden * 4, wbytes = (size_t)v16 * hidden * 2;
  const size_t tbytes = (size_t)n_target * 4;
  if (overlaps(target_ids, tbytes, h, hbytes) || overlaps(target_ids, tbytes, w_head, wbytes) ||
      overlaps(target_ids, tbytes, workspace, need) || overlaps(accepted, 4, h, hbytes) ||
      overlaps(accepted, 4, w_head, wbytes) || overlaps(accepted, 4, workspace, need) ||
      overlaps(accepted, 4, target_ids, tbytes) || overlaps(workspace, need, h, hbytes) ||
      overlaps(workspace, need, w_head, wbytes))
    return MOE_ERR_ALIAS;
  const int G = std::min(num_cus(), HEAD_GMAX);
  const int n_items = (int)((v16 / 16 + 1) / 2);
  const size_t part = align256((size_t)n_target * HEAD_GMAX * 4);
  float* pv = (float*)workspace;
  int* pi = (int*)((uint8_t*)workspace + part);
  uint64_t* ctr = (uint64_t*)((uint8_t*)workspace + 2 * part);
  // a fresh epoch per call tags this call's claim pools (zero is never used)
  static std::atomic<uint32_t> calls{0};
  uint32_t epoch = ++calls;
  if (epoch == 0) epoch = ++calls;
  hipStream_t s = (hipStream_t)hip_stream;
  if (error_pending()) return MOE_ERR_HIP;  // the caller's own error stays pending
  const uint8_t* w = (const uint8_t*)w_head;
  if (hidden <= NW * WIN) k_head<1><<<G, NTH, 0, s>>>(h, w, hidden, vocab, n_target, n_items, pv, pi, ctr, epoch);
  else                    k_head<2><<<G, NTH, 0, s>>>(h, w, hidden, vocab, n_target, n_items, pv, pi, ctr, epoch);
  k_accept_final<<<1, 1024, 0, s>>>(pv, pi, G, n_target, draft_ids, n_draft, target_ids, accepted);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// workspace: row partials ms [n_target + n_draft][nchunks] float2, chunk sums [nchunks] float2,
// the plan
size_t accept_sample_workspace_size(int32_t n_target, int32_t n_draft, int32_t vocab) {
  if (n_target < 1 || n_target > 64 || n_draft < 0 || n_draft > n_target || vocab < 1 || vocab > (1 << 24)) return 0;
  const size_t nch = ((size_t)vocab + AM_CHUNK - 1) / AM_CHUNK;
  return align256((size_t)(n_target + n_draft) * nch * 8) + align256(nch * 8) + align256(sizeof(SamplePlan));
}

int accept_sample(const float* target_logits, int32_t n_target, int32_t vocab, const float* draft_logits,
                  const int32_t* draft_ids, int32_t n_draft, float temperature, const float* u_accept,
                  const float* u_sample, int32_t* accepted, int32_t* token, void* workspace, size_t ws_bytes,
                  void* hip_stream) {
  if (!target_logits || !u_sample || !accepted || !token || !workspace ||
      (n_draft > 0 && (!draft_logits || !draft_ids || !u_accept)))
    return MOE_ERR_NULL;
  if (n_target < 1 || n_target > 64 || n_draft < 0 || n_draft > n_target || vocab < 1 || vocab > (1 << 24) ||
      !(temperature > 0.f) || !(temperature < INFINITY))
    return MOE_ERR_SHAPE;
  if (!aligned16(target_logits) || (draft_logits && !aligned16(draft_logits)) || !aligned16(workspace) ||
      (draft_ids && !aligned4(draft_ids)) || (u_accept && !aligned4(u_accept)) || !aligned4(u_sample) ||
      !aligned4(accepted) || !aligned4(token))
    return MOE_ERR_ALIGN;
  const size_t need = accept_sample_workspace_size(n_target, n_draft, vocab);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  const size_t tb = (size_t)n_target * vocab * 4, db = (size_t)n_draft * vocab * 4;
  const void* outs[3] = {accepted, token, workspace};
  const size_t osz[3] = {4, 4, need};
  const void* ins[5] = {target_logits, draft_logits, draft_ids, u_accept, u_sample};
  const size_t isz[5] = {tb, db, (size_t)n_draft * 4, (size_t)n_draft * 4, (size_t)n_target * 4};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 5; ++i)
      if (ins[i] && overlaps(outs[o], osz[o], ins[i], isz[i])) return MOE_ERR_ALIAS;
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlaps(outs[o], osz[o], outs[o2], osz[o2])) return MOE_ERR_ALIAS;
  }
  const int nch = (vocab + AM_CHUNK - 1) / AM_CHUNK;
  uint8_t* ws = (uint8_t*)workspace;
  float2* ms = (float2*)ws;
  float2* csum = (float2*)(ws + align256((size_t)(n_target + n_draft) * nch * 8));
  SamplePlan* plan = (SamplePlan*)(ws + align256((size_t)(n_target + n_draft) * nch * 8) + align256((size_t)nch * 8));
  const float zscale = 1.4426950408889634f / temperature;  // log2(e) / T
  hipStream_t s = (hipStream_t)hip_stream;
  if (error_pending()) return MOE_ERR_HIP;  // the caller's own error stays pending
  k_lse_partial<<<dim3(nch, n_target + n_draft), 256, 0, s>>>(target_logits, draft_logits, n_target, vocab, nch,
                                                             zscale, ms);
  k_sample_partial<<<nch, SAMPLE_NTH, 0, s>>>(target_logits, draft_logits, n_target, vocab, nch, zscale, draft_ids,
                                              n_draft, u_accept, u_sample, ms, csum, plan, accepted, token);
  k_sample_final<<<1, SAMPLE_NTH, 0, s>>>(target_logits, draft_logits, vocab, nch, zscale, csum, plan, token);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

size_t accept_sample_batch_workspace_size(int32_t n_seq, int32_t n_target, int32_t n_draft, int32_t vocab) {
  if (n_seq < 1 || n_seq > 1024) return 0;
  const size_t one = accept_sample_workspace_size(n_target, n_draft, vocab);
  if (!one) return 0;
  const size_t nch = ((size_t)vocab + AM_CHUNK - 1) / AM_CHUNK;
  return align256((size_t)n_seq * (n_target + n_draft) * nch * 8) + align256((size_t)n_seq * nch * 8) +
         align256((size_t)n_seq * sizeof(SamplePlan));
}

int accept_sample_batch(const float* target_logits, int32_t n_seq, int32_t n_target, int32_t vocab,
                        const float* draft_logits, const int32_t* draft_ids, int32_t n_draft, float temperature,
                        const float* u_accept, const float* u_sample, int32_t* accepted, int32_t* token,
                        void* workspace, size_t ws_bytes, void* hip_stream) {
  if (!target_logits || !u_sample || !accepted || !token || !workspace ||
      (n_draft > 0 && (!draft_logits || !draft_ids || !u_accept)))
    return MOE_ERR_NULL;
  if (n_seq < 1 || n_seq > 1024 || n_target < 1 || n_target > 64 || n_draft < 0 || n_draft > n_target ||
      vocab < 1 || vocab > (1 << 24) || !(temperature > 0.f) || !(temperature < INFINITY))
    return MOE_ERR_SHAPE;
  if (!aligned16(target_logits) || (draft_logits && !aligned16(draft_logits)) || !aligned16(workspace) ||
      (draft_ids && !aligned4(draft_ids)) || (u_accept && !aligned4(u_accept)) || !aligned4(u_sample) ||
      !aligned4(accepted) || !aligned4(token))
    return MOE_ERR_ALIGN;
  const size_t need = accept_sample_batch_workspace_size(n_seq, n_target, n_draft, vocab);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  const size_t S = (size_t)n_seq;
  const size_t tb = S * n_target * vocab * 4, db = S * n_draft * vocab * 4;
  const void* outs[3] = {accepted, token, workspace};
  const size_t osz[3] = {S * 4, S * 4, need};
  const void* ins[5] = {target_logits, draft_logits, draft_ids, u_accept, u_sample};
  const size_t isz[5] = {tb, db, S * n_draft * 4, S * n_draft * 4, S * n_target * 4};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 5; ++i)
      if (ins[i] && overlaps(outs[o], osz[o], ins[i], isz[i])) return MOE_ERR_ALIAS;
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlaps(outs[o], osz[o], outs[o2], osz[o2])) return MOE_ERR_ALIAS;
  }
  const int nch = (vocab + AM_CHUNK - 1) / AM_CHUNK;
  uint8_t* ws = (uint8_t*)workspace;
  const size_t b0 = align256(S * (n_target + n_draft) * nch * 8), b1 = align256(S * nch * 8);
  float2* ms = (float2*)ws;
  float2* csum = (float2*)(ws + b0);
  SamplePlan* plan = (SamplePlan*)(ws + b0 + b1);
  const float zscale = 1.4426950408889634f / temperature;  // log2(e) / T
  hipStream_t s = (hipStream_t)hip_stream;
  if (error_pending()) return MOE_ERR_HIP;  // the caller's own error stays pending
  k_lse_partial<<<dim3(nch, n_target + n_draft, n_seq), 256, 0, s>>>(target_logits, draft_logits, n_target, vocab,
                                                                     nch, zscale, ms);
  k_sample_partial<<<dim3(nch, n_seq), SAMPLE_NTH, 0, s>>>(target_logits, draft_logits, n_target, vocab, nch,
                                                           zscale, draft_ids, n_draft, u_accept, u_sample, ms, csum,
                                                           plan, accepted, token);
  k_sample_final<<<n_seq, SAMPLE_NTH, 0, s>>>(target_logits, draft_logits, vocab, nch, zscale, csum, plan, token,
                                              n_target, n_draft);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int accept_histogram(const int32_t* accepted, int32_t n_cycles, int32_t n_draft, int64_t* hist, int64_t* survival,
                     void* hip_stream) {
  if (!accepted || !hist || (n_draft > 0 && !survival)) return MOE_ERR_NULL;
  if (n_cycles < 0 || n_draft < 0 || n_draft > 64) return MOE_ERR_SHAPE;
  if (!aligned4(accepted) || !aligned8(hist) || (survival && !aligned8(survival))) return MOE_ERR_ALIGN;
  const size_t ab = (size_t)n_cycles * 4, hb = (size_t)(n_draft + 1) * 8, sb = (size_t)n_draft * 8;
  if (overlaps(hist, hb, accepted, ab) || (survival && (overlaps(survival, sb, accepted, ab) ||
                                                        overlaps(survival, sb, hist, hb))))
    return MOE_ERR_ALIAS;
  if (error_pending()) return MOE_ERR_HIP;  // the caller's own error stays pending
  k_accept_hist<<<1, 1024, 0, (hipStream_t)hip_stream>>>(accepted, n_cycles, n_draft, hist, survival);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
