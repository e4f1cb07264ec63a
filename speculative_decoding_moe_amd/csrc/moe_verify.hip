// MoE verify-block library for gfx950 (CDNA4). C ABI in include/moe_verify.h.
//
// One MoE layer over a speculative block of k <= 16 tokens ("Speculating on a Strix Halo",
// sections "Speculative decoding", "What the pieces cost", "The verify's own cost"), in four
// launches on the caller's stream:
//
//   k_router   fp32 router GEMV for all block tokens (W_r read once), optional RMSNorm, and the
//              normalised block packed as bf16 hi/lo MFMA B-operand fragments.
//   k_gateup   per workgroup: top-K + softmax per token and the woken-expert union (LDS, wave
//              ballot + prefix count), then a grid-stride loop over (woken expert, row tile)
//              items: each woken expert's gate/up rows are streamed from HBM exactly once
//              (128-bit nontemporal loads) and applied to the whole block with MFMA; the SwiGLU
//              epilogue scales by the routing weight and writes the down projection's B operand.
//   k_down     grid-stride loop over (woken expert, row group) items: W_down streamed once, MFMA
//              against that expert's activations, per-(token, slot) partial rows.
//   k_combine  y[t] = sum_j P[t, j] + P[t, shared] (+ x[t]) in fixed order.
//
// Tokens are the MFMA N dimension (16 columns; unused columns are explicit zeros written every
// call), expert rows the M dimension, the hidden / intermediate size the K dimension. MFMA work
// is free next to the HBM stream, so every expert is applied to all 16 columns and columns of
// tokens not routed to it carry weight 0. Activations enter MFMA as a bf16 hi + lo pair, which
// keeps the products at ~2^-17 relative precision at the cost of a second MFMA per tile.
//
// K-index mapping used by every MFMA tile: the reduction dimension is cut into windows of 128;
// in window w, k-step j (0..3), lane l = c + 16 q (c = row or token column, q = 0..3) holds the
// 8 values at offsets 128 w + 32 q + 8 j + (0..7). A lane's four k-steps of one window are 64
// contiguous bf16 bytes, or one 32-value mxfp4 block with a single scale byte.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "moe_verify.h"

namespace {

constexpr int KMAX = 16;       // block tokens = MFMA N
constexpr int WIN = 128;       // reduction window
constexpr int GU_WAVES = 8;    // gate/up workgroup = 512 threads, WPW 128-windows of H per wave
constexpr int DN_WAVES = 4;    // down workgroup = 256 threads
constexpr int RT_EPB = 4;      // router: experts per workgroup
constexpr int MAX_E = 512;
constexpr int MAX_K = 16;
constexpr int GU_MX_RT = 2;    // gate/up row tiles per mxfp4 item (bf16 items: 1)
constexpr int DN_RT_BF = 8;    // down row tiles per bf16 item (divided by windows per wave)
constexpr int DN_RT_MX = 16;   // down row tiles per mxfp4 item (divided by windows per wave)
constexpr int AM_CHUNK = 8192; // argmax values per workgroup

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Weights are read once per call: nontemporal 128-bit loads.
__device__ __forceinline__ u32x4 ld_stream(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}
__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }

__device__ __forceinline__ uint32_t bf16_rne(float f) {  // finite inputs
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// f ~= hi + lo with both halves bf16.
__device__ __forceinline__ void split_bf16(float f, uint32_t& hi, uint32_t& lo) {
  hi = bf16_rne(f);
  lo = bf16_rne(f - __uint_as_float(hi << 16));
}

// Eight E2M1 codes (one dword, element 2j in the low nibble of byte j) -> eight bf16 scaled by
// `scale` (a power of two built from the e8m0 byte).
__device__ __forceinline__ u32x4 dec_fp4x8(uint32_t c, float scale) {
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 3));
  return r;
}
__device__ __forceinline__ float e8m0_scale(uint32_t byte) { return __uint_as_float(byte << 23); }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

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
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// ------------------------------------------------------------------------------------------
// workspace layout (host and device agree through the offsets passed in the kernel args)
// ------------------------------------------------------------------------------------------
struct Layout {
  size_t xfrag, logits, tab_n, tab_woken, tab_slot, afrag, afrag_sh, part, total;
  int umax;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

Layout make_layout(const moe_layer* L, int k) {
  Layout o;
  const size_t H = L->hidden, E = L->n_experts, K = L->top_k, I = L->inter, Is = L->shared_inter;
  o.umax = (int)((E < (size_t)KMAX * K) ? E : (size_t)KMAX * K);
  size_t off = 0;
  o.xfrag = off;     off = align256(off + H * 64);               // (H/32) k-steps x hi/lo x 64 lanes x 16 B
  o.logits = off;    off = align256(off + (size_t)KMAX * E * 4);
  o.tab_n = off;     off = align256(off + 16);
  o.tab_woken = off; off = align256(off + (size_t)o.umax * 4);
  o.tab_slot = off;  off = align256(off + (size_t)o.umax * KMAX);
  o.afrag = off;     off = align256(off + (size_t)o.umax * I * 64);
  o.afrag_sh = off;  off = align256(off + Is * 64);
  o.part = off;      off = align256(off + (size_t)k * (K + 1) * H * 4);
  o.total = off;
  return o;
}

// ------------------------------------------------------------------------------------------
// k_router: logits[t][e] = rinv_t * sum_h x[t][h] W_r[e][h]  (fp32), rinv_t = 1 or the RMSNorm
// factor; also packs x_hat = rinv_t * x[t] into the gate/up B-operand fragments.
// ------------------------------------------------------------------------------------------
struct RouterArgs {
  const float* x;
  const float* wr;
  float* logits;
  u32x4* xfrag;
  int H, E, k;
  int pre_norm;
  float eps;
};

constexpr int RT_THREADS = 256;
constexpr int RT_MAXC = 2048 / 4 / RT_THREADS;  // float4 chunks per thread per row (H <= 2048)

__global__ void __launch_bounds__(RT_THREADS) k_router(RouterArgs a) {
  __shared__ float s_part[RT_THREADS / 64][KMAX * (RT_EPB + 1)];
  __shared__ float s_rinv[KMAX];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int H4 = a.H / 4, k = a.k;
  const int e0 = blockIdx.x * RT_EPB;

  float4 w[RT_EPB][RT_MAXC];
#pragma unroll
  for (int e = 0; e < RT_EPB; ++e)
#pragma unroll
    for (int c = 0; c < RT_MAXC; ++c) {
      int col = tid + c * RT_THREADS;
      w[e][c] = (e0 + e < a.E && col < H4)
                    ? reinterpret_cast<const float4*>(a.wr + (size_t)(e0 + e) * a.H)[col]
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }

  float acc[KMAX][RT_EPB + 1];  // [.][RT_EPB] holds the sum of squares
#pragma unroll
  for (int t = 0; t < KMAX; ++t) {
#pragma unroll
    for (int e = 0; e <= RT_EPB; ++e) acc[t][e] = 0.f;
    if (t < k) {
#pragma unroll
      for (int c = 0; c < RT_MAXC; ++c) {
        int col = tid + c * RT_THREADS;
        if (col < H4) {
          float4 xv = reinterpret_cast<const float4*>(a.x + (size_t)t * a.H)[col];
#pragma unroll
          for (int e = 0; e < RT_EPB; ++e)
            acc[t][e] += w[e][c].x * xv.x + w[e][c].y * xv.y + w[e][c].z * xv.z + w[e][c].w * xv.w;
          acc[t][RT_EPB] += xv.x * xv.x + xv.y * xv.y + xv.z * xv.z + xv.w * xv.w;
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < KMAX; ++t)
#pragma unroll
    for (int e = 0; e <= RT_EPB; ++e) {
      float v = wave_sum(acc[t][e]);
      if (lane == 0) s_part[wave][t * (RT_EPB + 1) + e] = v;
    }
  __syncthreads();
  if (tid < KMAX * (RT_EPB + 1)) {
    float v = 0.f;
#pragma unroll
    for (int wv = 0; wv < RT_THREADS / 64; ++wv) v += s_part[wv][tid];
    s_part[0][tid] = v;
  }
  __syncthreads();
  if (tid < KMAX) {
    float ss = s_part[0][tid * (RT_EPB + 1) + RT_EPB];
    s_rinv[tid] = a.pre_norm ? 1.0f / sqrtf(ss / (float)a.H + a.eps) : 1.0f;
  }
  __syncthreads();
  if (tid < k * RT_EPB) {
    int t = tid / RT_EPB, e = tid % RT_EPB;
    if (e0 + e < a.E) a.logits[(size_t)t * a.E + e0 + e] = s_rinv[t] * s_part[0][t * (RT_EPB + 1) + e];
  }
  // B-operand fragments of x_hat: k-steps s = blockIdx.x, blockIdx.x + gridDim.x, ...
  const int nsteps = a.H / 32;
  for (int s = blockIdx.x; s < nsteps; s += gridDim.x) {
    if (tid < 64) {
      const int t = tid & 15, q = tid >> 4, w = s >> 2, j = s & 3;
      uint32_t hi[8], lo[8];
      if (t < k) {
        const float* src = a.x + (size_t)t * a.H + w * WIN + 32 * q + 8 * j;
        float4 v0 = *reinterpret_cast<const float4*>(src);
        float4 v1 = *reinterpret_cast<const float4*>(src + 4);
        float r = s_rinv[t];
        float f[8] = {v0.x * r, v0.y * r, v0.z * r, v0.w * r, v1.x * r, v1.y * r, v1.z * r, v1.w * r};
#pragma unroll
        for (int i = 0; i < 8; ++i) split_bf16(f[i], hi[i], lo[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) hi[i] = lo[i] = 0u;
      }
      u32x4 h, l;
      h.x = hi[0] | (hi[1] << 16); h.y = hi[2] | (hi[3] << 16); h.z = hi[4] | (hi[5] << 16); h.w = hi[6] | (hi[7] << 16);
      l.x = lo[0] | (lo[1] << 16); l.y = lo[2] | (lo[3] << 16); l.z = lo[4] | (lo[5] << 16); l.w = lo[6] | (lo[7] << 16);
      a.xfrag[((size_t)s * 2 + 0) * 64 + tid] = h;
      a.xfrag[((size_t)s * 2 + 1) * 64 + tid] = l;
    }
  }
}

// ------------------------------------------------------------------------------------------
// k_gateup: routing prologue, then (woken expert, row tile) items. Wave w owns H-window w.
// ------------------------------------------------------------------------------------------
struct GUArgs {
  const float* logits;
  const u32x4* xfrag;
  const uint8_t* wg;   // routed gate (bf16 or fp4 codes)
  const uint8_t* wu;
  const uint8_t* sg;   // routed scales (mxfp4)
  const uint8_t* su;
  const uint8_t* shg;  // shared gate/up (bf16)
  const uint8_t* shu;
  u32x4* afrag;
  u32x4* afrag_sh;
  int32_t* tab_n;
  int32_t* tab_woken;
  int8_t* tab_slot;
  int32_t* out_ids;
  float* out_w;
  int32_t* out_n;
  int H, E, K, I, Is, k;
};

// One item's weights for one wave (its WPW windows of H).
//   bf16 item:  v[(wi * 2 + mat) * 4 + j] = 8 values of k-step j     (64 B per lane, window, matrix)
//   mxfp4 item: v[(tile * WPW + wi) * 2 + mat] = 32 codes, sc[...] = their e8m0 scale byte
template <int WPW>
struct GUItem {
  u32x4 v[WPW * 8];
  uint32_t sc[GU_MX_RT * WPW * 2];
};

struct GUDesc {
  int routed, u, row0, mx, ntile;
  const uint8_t* g;
  const uint8_t* up;
  const uint8_t* sg;
  const uint8_t* su;
};

__device__ __forceinline__ GUDesc gu_desc(const GUArgs& a, int item, int n_routed, int ipe, int U,
                                          const int* woken, bool MX) {
  GUDesc d;
  d.routed = item < n_routed;
  d.u = d.routed ? item / ipe : U;
  d.mx = MX && d.routed;
  d.ntile = d.mx ? GU_MX_RT : 1;
  d.row0 = (d.routed ? item % ipe : item - n_routed) * 16 * d.ntile;
  const size_t H = a.H, I = a.I;
  if (d.routed) {
    const size_t e = (size_t)__builtin_amdgcn_readfirstlane(woken[d.u]);
    if (d.mx) {
      d.g = a.wg + e * I * (H / 2); d.up = a.wu + e * I * (H / 2);
      d.sg = a.sg + e * I * (H / 32); d.su = a.su + e * I * (H / 32);
    } else {
      d.g = a.wg + e * I * H * 2; d.up = a.wu + e * I * H * 2;
      d.sg = d.su = nullptr;
    }
  } else {
    d.g = a.shg; d.up = a.shu; d.sg = d.su = nullptr;
  }
  return d;
}

template <int WPW>
__device__ __forceinline__ void gu_load(GUItem<WPW>& T, const GUDesc& d, int H, int win0, int lane) {
  const int q = lane >> 4, r = lane & 15;
  if (d.mx) {
    const size_t base = ((size_t)d.row0 + r) * (H / 2) + (size_t)win0 * 64 + 16 * q;
    const size_t sbase = ((size_t)d.row0 + r) * (H / 32) + (size_t)win0 * 4 + q;
#pragma unroll
    for (int tl = 0; tl < GU_MX_RT; ++tl)
#pragma unroll
      for (int wi = 0; wi < WPW; ++wi) {
        const size_t off = base + (size_t)tl * 16 * (H / 2) + wi * 64;
        const size_t soff = sbase + (size_t)tl * 16 * (H / 32) + wi * 4;
        T.v[(tl * WPW + wi) * 2 + 0] = ld_stream(d.g + off);
        T.v[(tl * WPW + wi) * 2 + 1] = ld_stream(d.up + off);
        T.sc[(tl * WPW + wi) * 2 + 0] = d.sg[soff];
        T.sc[(tl * WPW + wi) * 2 + 1] = d.su[soff];
      }
  } else {
    const size_t off = (((size_t)d.row0 + r) * H + (size_t)win0 * WIN + 32 * q) * 2;
#pragma unroll
    for (int wi = 0; wi < WPW; ++wi)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        T.v[(wi * 2 + 0) * 4 + j] = ld_stream(d.g + off + wi * WIN * 2 + 16 * j);
        T.v[(wi * 2 + 1) * 4 + j] = ld_stream(d.up + off + wi * WIN * 2 + 16 * j);
      }
  }
}

struct alignas(16) GUShared {
  float red[GU_WAVES][GU_MX_RT][2][256];  // per-wave partial tiles
  float act[GU_MX_RT][256];               // reduced, activated tiles
  int ids[KMAX][MAX_K];
  float val[KMAX][MAX_K];
  float w[KMAX][MAX_K];
  uint8_t flag[MAX_E];
  int pos[MAX_E];
  int woken[KMAX * MAX_K];
  float wcol[KMAX * MAX_K + 1][KMAX];
  int8_t slot[KMAX * MAX_K][KMAX];
  int nw;
};

// MFMA of one item, cross-wave reduction, SwiGLU, weight, hi/lo split, store as down-projection
// B fragments. Contains two workgroup barriers.
template <int WPW>
__device__ __forceinline__ void gu_process(const GUArgs& a, GUShared& S, const GUItem<WPW>& T,
                                           const GUDesc& d, const u32x4 (&xb)[WPW][4][2], bool active,
                                           int wave, int lane, int tid) {
  f32x4 acc[GU_MX_RT][2];
#pragma unroll
  for (int tl = 0; tl < GU_MX_RT; ++tl) acc[tl][0] = acc[tl][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (active) {
    if (d.mx) {
#pragma unroll
      for (int tl = 0; tl < GU_MX_RT; ++tl)
#pragma unroll
        for (int wi = 0; wi < WPW; ++wi)
#pragma unroll
          for (int mat = 0; mat < 2; ++mat) {
            const u32x4 c = T.v[(tl * WPW + wi) * 2 + mat];
            const float sc = e8m0_scale(T.sc[(tl * WPW + wi) * 2 + mat]);
            const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const u32x4 av = dec_fp4x8(cw[j], sc);
              acc[tl][mat] = mfma16(av, xb[wi][j][0], acc[tl][mat]);
              acc[tl][mat] = mfma16(av, xb[wi][j][1], acc[tl][mat]);
            }
          }
    } else {
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
  }
  // D[r][c] of a tile: lane c + 16 (r / 4), element r % 4  ->  red[...][lane * 4 + element]
#pragma unroll
  for (int tl = 0; tl < GU_MX_RT; ++tl)
    if (tl < d.ntile) {
      *reinterpret_cast<f32x4*>(&S.red[wave][tl][0][lane * 4]) = acc[tl][0];
      *reinterpret_cast<f32x4*>(&S.red[wave][tl][1][lane * 4]) = acc[tl][1];
    }
  __syncthreads();
  for (int i = tid; i < d.ntile * 256; i += GU_WAVES * 64) {
    const int tl = i >> 8, p = i & 255;
    float g = 0.f, up = 0.f;
#pragma unroll
    for (int wv = 0; wv < GU_WAVES; ++wv) {
      g += S.red[wv][tl][0][p];
      up += S.red[wv][tl][1][p];
    }
    const int c = (p >> 2) & 15;
    S.act[tl][p] = silu(g) * up * S.wcol[d.u][c];
  }
  __syncthreads();
  // thread (tile, half, column c) -> rows R .. R+7 of the expert's intermediate dimension
  if (tid < d.ntile * 2 * KMAX) {
    const int tl = tid / (2 * KMAX), half = (tid / KMAX) & 1, c = tid % KMAX;
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = half * 8 + i;
      split_bf16(S.act[tl][(c + 16 * (r >> 2)) * 4 + (r & 3)], hi[i], lo[i]);
    }
    const int R = d.row0 + 16 * tl + 8 * half;
    const int w = R / WIN, q = (R % WIN) / 32, j = (R % 32) / 8;
    const int s = w * 4 + j;
    u32x4* dst = d.routed ? a.afrag + (size_t)d.u * (a.I / 32) * 128 : a.afrag_sh;
    u32x4 h, l;
    h.x = hi[0] | (hi[1] << 16); h.y = hi[2] | (hi[3] << 16); h.z = hi[4] | (hi[5] << 16); h.w = hi[6] | (hi[7] << 16);
    l.x = lo[0] | (lo[1] << 16); l.y = lo[2] | (lo[3] << 16); l.z = lo[4] | (lo[5] << 16); l.w = lo[6] | (lo[7] << 16);
    dst[((size_t)s * 2 + 0) * 64 + c + 16 * q] = h;
    dst[((size_t)s * 2 + 1) * 64 + c + 16 * q] = l;
  }
}

template <int WPW, bool MX>
__global__ void __launch_bounds__(GU_WAVES * 64) k_gateup(GUArgs a) {
  __shared__ GUShared S;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int E = a.E, K = a.K, k = a.k, H = a.H;
  // H is a multiple of 128 * WPW, so a wave's windows all exist or none does
  const int win0 = wave * WPW;
  const bool active = win0 < H / WIN;

  // B fragments of this wave's windows, used by every item.
  u32x4 xb[WPW][4][2];
#pragma unroll
  for (int wi = 0; wi < WPW; ++wi)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl)
        xb[wi][j][hl] = active ? ld16(a.xfrag + ((size_t)((win0 + wi) * 4 + j) * 2 + hl) * 64 + lane)
                               : u32x4{0u, 0u, 0u, 0u};

  // ---- routing: top-K per token (one wave per token), softmax over the K, union ----
  for (int i = tid; i < MAX_E; i += GU_WAVES * 64) S.flag[i] = 0;
  for (int t = wave; t < k; t += GU_WAVES) {
    float v[MAX_E / 64];
    uint32_t taken = 0;
#pragma unroll
    for (int m = 0; m < MAX_E / 64; ++m) {
      const int e = lane + 64 * m;
      v[m] = (e < E) ? a.logits[(size_t)t * E + e] : 0.f;
      if (e >= E) taken |= 1u << m;
    }
    for (int j = 0; j < K; ++j) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int m = 0; m < MAX_E / 64; ++m)
        if (!((taken >> m) & 1u)) argmax_merge(bv, bi, v[m], lane + 64 * m);
      wave_argmax(bv, bi);
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      if (lane == 0) { S.ids[t][j] = bi; S.val[t][j] = bv; }
    }
  }
  __syncthreads();
  if (tid < k) {
    const int t = tid;
    const float m = S.val[t][0];
    float sum = 0.f;
    for (int j = 0; j < K; ++j) sum += expf(S.val[t][j] - m);
    for (int j = 0; j < K; ++j) S.w[t][j] = expf(S.val[t][j] - m) / sum;
  }
  if (tid < k * K) S.flag[S.ids[tid / K][tid % K]] = 1;
  __syncthreads();
  if (wave == 0) {
    int base = 0;
    for (int c = 0; c < (E + 63) / 64; ++c) {
      const int e = c * 64 + lane;
      const bool f = e < E && S.flag[e];
      const unsigned long long m = __ballot(f);
      const int p = base + __popcll(m & ((1ull << lane) - 1ull));
      if (f) { S.woken[p] = e; S.pos[e] = p; }
      base += __popcll(m);
    }
    if (lane == 0) S.nw = base;
  }
  __syncthreads();
  const int U = __builtin_amdgcn_readfirstlane(S.nw);
  for (int i = tid; i < (U + 1) * KMAX; i += GU_WAVES * 64) {
    S.wcol[i / KMAX][i % KMAX] = 0.f;
    if (i < U * KMAX) S.slot[i / KMAX][i % KMAX] = -1;
  }
  __syncthreads();
  if (tid < k * K) {
    const int t = tid / K, j = tid % K;
    const int u = S.pos[S.ids[t][j]];
    S.wcol[u][t] = S.w[t][j];
    S.slot[u][t] = (int8_t)j;
  }
  if (tid < KMAX) S.wcol[U][tid] = (tid < k) ? 1.0f : 0.f;  // shared expert column weights
  __syncthreads();
  if (blockIdx.x == 0) {
    if (tid < k * K) {
      const int t = tid / K, j = tid % K;
      if (a.out_ids) a.out_ids[t * K + j] = S.ids[t][j];
      if (a.out_w) a.out_w[t * K + j] = S.w[t][j];
    }
    if (tid == 0) {
      a.tab_n[0] = U;
      if (a.out_n) a.out_n[0] = U;
    }
    for (int i = tid; i < U; i += GU_WAVES * 64) a.tab_woken[i] = S.woken[i];
    for (int i = tid; i < U * KMAX; i += GU_WAVES * 64) a.tab_slot[i] = S.slot[i / KMAX][i % KMAX];
  }

  // ---- expert items, next item's weights prefetched while the current one is reduced ----
  const int ipe = a.I / (16 * (MX ? GU_MX_RT : 1));  // items per routed expert
  const int n_routed = U * ipe;
  const int n_items = n_routed + a.Is / 16;
  int item = blockIdx.x;
  GUItem<WPW> T0, T1;
  GUDesc d0, d1;
  if (item < n_items) {
    d0 = gu_desc(a, item, n_routed, ipe, U, S.woken, MX);
    if (active) gu_load<WPW>(T0, d0, H, win0, lane);
  }
  while (item < n_items) {
    int nxt = item + gridDim.x;
    if (nxt < n_items) {
      d1 = gu_desc(a, nxt, n_routed, ipe, U, S.woken, MX);
      if (active) gu_load<WPW>(T1, d1, H, win0, lane);
    }
    __builtin_amdgcn_sched_barrier(0);  // the next item's loads stay ahead of this item's math
    gu_process<WPW>(a, S, T0, d0, xb, active, wave, lane, tid);
    item = nxt;
    if (item >= n_items) break;
    nxt = item + gridDim.x;
    if (nxt < n_items) {
      d0 = gu_desc(a, nxt, n_routed, ipe, U, S.woken, MX);
      if (active) gu_load<WPW>(T0, d0, H, win0, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    gu_process<WPW>(a, S, T1, d1, xb, active, wave, lane, tid);
    item = nxt;
  }
}

// ------------------------------------------------------------------------------------------
// k_down: P[t][slot][h] = sum_i W_down[e][h][i] * A'[e][t][i] for tokens routed to e.
// Wave w owns I-windows w*WPWD .. w*WPWD+WPWD-1; an item is (woken expert, group of row tiles).
// ------------------------------------------------------------------------------------------
struct DNArgs {
  const u32x4* afrag;
  const u32x4* afrag_sh;
  const uint8_t* wd;
  const uint8_t* sd;
  const uint8_t* shd;
  const int32_t* tab_n;
  const int32_t* tab_woken;
  const int8_t* tab_slot;
  float* part;
  int H, E, K, I, Is, k;
};

template <int WPWD, bool MX>
__global__ void __launch_bounds__(DN_WAVES * 64) k_down(DNArgs a) {
  constexpr int RT_BF = DN_RT_BF / WPWD;  // row tiles per bf16 item
  constexpr int RT_MX = DN_RT_MX / WPWD;  // row tiles per mxfp4 item
  constexpr int RT_ACC = MX ? RT_MX : RT_BF;
  __shared__ __attribute__((aligned(16))) float red[DN_WAVES][RT_ACC][256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int H = a.H, I = a.I, K = a.K, k = a.k;
  const int U = a.tab_n[0];
  const int ipe = H / (16 * (MX ? RT_MX : RT_BF));
  const int n_routed = U * ipe;
  const int n_items = n_routed + (a.Is > 0 ? H / (16 * RT_BF) : 0);
  const int q = lane >> 4, r16 = lane & 15;
  // I (== Is when there is a shared expert) is 128 * 2^n, so a wave's WPWD windows all exist or
  // none does.
  const bool active = wave * WPWD < I / WIN;
  const int win0 = wave * WPWD;

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const bool routed = item < n_routed;
    const int u = routed ? item / ipe : U;
    const bool mx_item = MX && routed;
    const int ntile = mx_item ? RT_MX : RT_BF;
    const int row0 = (routed ? item % ipe : item - n_routed) * 16 * ntile;
    const u32x4* af = routed ? a.afrag + (size_t)u * (I / 32) * 128 : a.afrag_sh;

    f32x4 acc[RT_ACC];
#pragma unroll
    for (int tl = 0; tl < RT_ACC; ++tl) acc[tl] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (active) {
      u32x4 bf[WPWD][4][2];
#pragma unroll
      for (int wi = 0; wi < WPWD; ++wi)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int hl = 0; hl < 2; ++hl)
            bf[wi][j][hl] = ld16(af + ((size_t)((win0 + wi) * 4 + j) * 2 + hl) * 64 + lane);
      if (mx_item) {
        u32x4 v[RT_MX * WPWD];
        uint32_t sc[RT_MX * WPWD];
        const size_t e = (size_t)a.tab_woken[u];
        const uint8_t* w = a.wd + e * H * (I / 2) + (size_t)(row0 + r16) * (I / 2) + (size_t)win0 * 64 + 16 * q;
        const uint8_t* sw = a.sd + e * H * (I / 32) + (size_t)(row0 + r16) * (I / 32) + (size_t)win0 * 4 + q;
#pragma unroll
        for (int tl = 0; tl < RT_MX; ++tl)
#pragma unroll
          for (int wi = 0; wi < WPWD; ++wi) {
            v[tl * WPWD + wi] = ld_stream(w + (size_t)tl * 16 * (I / 2) + wi * 64);
            sc[tl * WPWD + wi] = sw[(size_t)tl * 16 * (I / 32) + wi * 4];
          }
        __builtin_amdgcn_sched_barrier(0);  // keep every load of the item ahead of the math
#pragma unroll
        for (int tl = 0; tl < RT_MX; ++tl)
#pragma unroll
          for (int wi = 0; wi < WPWD; ++wi) {
            const u32x4 c = v[tl * WPWD + wi];
            const float s = e8m0_scale(sc[tl * WPWD + wi]);
            const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const u32x4 av = dec_fp4x8(cw[j], s);
              acc[tl] = mfma16(av, bf[wi][j][0], acc[tl]);
              acc[tl] = mfma16(av, bf[wi][j][1], acc[tl]);
            }
          }
      } else {
        u32x4 v[RT_BF * WPWD * 4];
        const uint8_t* w = (routed ? a.wd + (size_t)a.tab_woken[u] * H * I * 2 : a.shd) +
                           ((size_t)(row0 + r16) * I + (size_t)win0 * WIN + 32 * q) * 2;
#pragma unroll
        for (int tl = 0; tl < RT_BF; ++tl)
#pragma unroll
          for (int wi = 0; wi < WPWD; ++wi)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              v[(tl * WPWD + wi) * 4 + j] = ld_stream(w + ((size_t)tl * 16 * I + wi * WIN) * 2 + 16 * j);
        __builtin_amdgcn_sched_barrier(0);  // keep every load of the item ahead of the math
#pragma unroll
        for (int tl = 0; tl < RT_BF; ++tl)
#pragma unroll
          for (int wi = 0; wi < WPWD; ++wi)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              acc[tl] = mfma16(v[(tl * WPWD + wi) * 4 + j], bf[wi][j][0], acc[tl]);
              acc[tl] = mfma16(v[(tl * WPWD + wi) * 4 + j], bf[wi][j][1], acc[tl]);
            }
      }
    }
#pragma unroll
    for (int tl = 0; tl < RT_ACC; ++tl)
      if (tl < ntile) *reinterpret_cast<f32x4*>(&red[wave][tl][lane * 4]) = acc[tl];
    __syncthreads();
    {
      const int r = tid & 15, c = tid >> 4;  // row within a tile, token column
      int slot = -1;
      if (c < k) slot = routed ? (int)a.tab_slot[u * KMAX + c] : K;
      if (slot >= 0) {
        float* dst = a.part + ((size_t)c * (K + 1) + slot) * H + row0 + r;
        const int idx = (c + 16 * (r >> 2)) * 4 + (r & 3);
        for (int tl = 0; tl < ntile; ++tl) {
          float v = 0.f;
#pragma unroll
          for (int wv = 0; wv < DN_WAVES; ++wv) v += red[wv][tl][idx];
          dst[tl * 16] = v;
        }
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------
// k_combine: y[t] = (sum_j P[t][j]) + P[t][K] (+ x[t]), fixed order
// ------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_combine(const float* part, const float* x, float* y, int H,
                                                 int K, int k, int has_shared, int residual) {
  const int H4 = H / 4;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= k * H4) return;
  const int t = idx / H4, c = idx % H4;
  const float4* p = reinterpret_cast<const float4*>(part + (size_t)t * (K + 1) * H) + c;
  float4 acc = p[0];
  for (int j = 1; j < K; ++j) {
    const float4 v = p[(size_t)j * H4];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  if (has_shared) {
    const float4 v = p[(size_t)K * H4];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  if (residual) {
    const float4 v = reinterpret_cast<const float4*>(x + (size_t)t * H)[c];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  reinterpret_cast<float4*>(y + (size_t)t * H)[c] = acc;
}

// ------------------------------------------------------------------------------------------
// accept_prefix kernels
// ------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_argmax_partial(const float* logits, int V, int nchunks,
                                                        float* pv, int* pi) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int row = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const int base = chunk * AM_CHUNK;
  const int end = min(base + AM_CHUNK, V);
  const float* r = logits + (size_t)row * V;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if ((V & 3) == 0) {
    for (int i = base + 4 * tid; i < end; i += 4 * 256) {
      const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r + i));
      argmax_merge(bv, bi, v.x, i);
      argmax_merge(bv, bi, v.y, i + 1);
      argmax_merge(bv, bi, v.z, i + 2);
      argmax_merge(bv, bi, v.w, i + 3);
    }
  } else {
    for (int i = base + tid; i < end; i += 256) argmax_merge(bv, bi, r[i], i);
  }
  wave_argmax(bv, bi);
  if ((tid & 63) == 0) { sv[tid >> 6] = bv; si[tid >> 6] = bi; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) argmax_merge(bv, bi, sv[w], si[w]);
    pv[(size_t)row * nchunks + chunk] = bv;
    pi[(size_t)row * nchunks + chunk] = bi;
  }
}

__global__ void __launch_bounds__(64) k_accept_final(const float* pv, const int* pi, int nchunks,
                                                     int n_target, const int32_t* draft, int n_draft,
                                                     int32_t* target_ids, int32_t* accepted) {
  __shared__ int tgt[64];
  const int tid = threadIdx.x;
  if (tid < n_target) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int c = 0; c < nchunks; ++c) argmax_merge(bv, bi, pv[(size_t)tid * nchunks + c], pi[(size_t)tid * nchunks + c]);
    tgt[tid] = bi;
    target_ids[tid] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    int a = 0;
    while (a < n_draft && draft[a] == tgt[a]) ++a;
    accepted[0] = a;
  }
}

// ------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

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
  if (I != 128 && I != 256 && I != 512 && I != 1024) return MOE_ERR_SHAPE;
  if (Is != 0 && Is != I) return MOE_ERR_SHAPE;
  if (L->wdtype != MOE_W_BF16 && L->wdtype != MOE_W_MXFP4) return MOE_ERR_DTYPE;
  if (L->wdtype == MOE_W_MXFP4 && H % 256) return MOE_ERR_SHAPE;  // mxfp4 down items are 256 rows
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

int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int WPW, bool MX>
void launch_gateup(const GUArgs& g, hipStream_t s, int grid) {
  k_gateup<WPW, MX><<<grid, GU_WAVES * 64, 0, s>>>(g);
}
template <int WPWD, bool MX>
void launch_down(const DNArgs& d, hipStream_t s, int grid) {
  k_down<WPWD, MX><<<grid, DN_WAVES * 64, 0, s>>>(d);
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is outside the supported range";
    case MOE_ERR_DTYPE: return "unknown weight format or missing mxfp4 scales";
    case MOE_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_ALIAS: return "an output overlaps an input";
    case MOE_ERR_HIP: return "kernel launch failed";
    case MOE_ERR_ARG: return "bad flag bits or scalar argument";
    default: return "unknown status";
  }
}

size_t moe_verify_workspace_size(const moe_layer* layer, int32_t k_max) {
  if (check_layer(layer) != MOE_OK || k_max < 1 || k_max > KMAX) return 0;
  return make_layout(layer, k_max).total;
}

static int verify_block_impl(const moe_layer* L, const float* x, int32_t k, uint32_t flags, float* y,
                             int32_t* topk_ids, float* topk_w, int32_t* n_woken, void* workspace,
                             size_t ws_bytes, void* hip_stream, void* const* events) {
  int st = check_layer(L);
  if (st != MOE_OK) return st;
  if (!x || !y || !workspace) return MOE_ERR_NULL;
  if (k < 1 || k > KMAX) return MOE_ERR_SHAPE;
  if (flags & ~(uint32_t)(MOE_PRE_RMSNORM | MOE_RESIDUAL)) return MOE_ERR_ARG;
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

  hipStream_t s = (hipStream_t)hip_stream;
  uint8_t* ws = (uint8_t*)workspace;
  const int H = L->hidden, E = L->n_experts;
  const bool mx = L->wdtype == MOE_W_MXFP4;

  (void)hipGetLastError();  // clear a stale error so the check below reports these launches
  auto mark = [&](int i) -> bool {
    return !events || !events[i] || hipEventRecord((hipEvent_t)events[i], s) == hipSuccess;
  };
  if (!mark(0)) return MOE_ERR_HIP;

  RouterArgs ra;
  ra.x = x; ra.wr = L->router_w; ra.logits = (float*)(ws + lay.logits); ra.xfrag = (u32x4*)(ws + lay.xfrag);
  ra.H = H; ra.E = E; ra.k = k; ra.pre_norm = (flags & MOE_PRE_RMSNORM) ? 1 : 0; ra.eps = L->rms_eps;
  k_router<<<(E + RT_EPB - 1) / RT_EPB, RT_THREADS, 0, s>>>(ra);
  if (!mark(1)) return MOE_ERR_HIP;

  GUArgs g;
  g.logits = ra.logits; g.xfrag = ra.xfrag;
  g.wg = (const uint8_t*)L->w_gate; g.wu = (const uint8_t*)L->w_up; g.sg = L->s_gate; g.su = L->s_up;
  g.shg = (const uint8_t*)L->sh_gate; g.shu = (const uint8_t*)L->sh_up;
  g.afrag = (u32x4*)(ws + lay.afrag); g.afrag_sh = (u32x4*)(ws + lay.afrag_sh);
  g.tab_n = (int32_t*)(ws + lay.tab_n); g.tab_woken = (int32_t*)(ws + lay.tab_woken);
  g.tab_slot = (int8_t*)(ws + lay.tab_slot);
  g.out_ids = topk_ids; g.out_w = topk_w; g.out_n = n_woken;
  g.H = H; g.E = E; g.K = L->top_k; g.I = L->inter; g.Is = L->shared_inter; g.k = k;
  const int cus = num_cus();
  if (H > 1024) { if (mx) launch_gateup<2, true>(g, s, cus); else launch_gateup<2, false>(g, s, cus); }
  else          { if (mx) launch_gateup<1, true>(g, s, cus); else launch_gateup<1, false>(g, s, cus); }
  if (!mark(2)) return MOE_ERR_HIP;

  DNArgs d;
  d.afrag = g.afrag; d.afrag_sh = g.afrag_sh;
  d.wd = (const uint8_t*)L->w_down; d.sd = L->s_down; d.shd = (const uint8_t*)L->sh_down;
  d.tab_n = g.tab_n; d.tab_woken = g.tab_woken; d.tab_slot = g.tab_slot;
  d.part = (float*)(ws + lay.part);
  d.H = H; d.E = E; d.K = L->top_k; d.I = L->inter; d.Is = L->shared_inter; d.k = k;
  const int wpwd = L->inter == 1024 ? 2 : 1;
  if (wpwd == 1) { if (mx) launch_down<1, true>(d, s, 2 * cus); else launch_down<1, false>(d, s, 2 * cus); }
  else           { if (mx) launch_down<2, true>(d, s, 2 * cus); else launch_down<2, false>(d, s, 2 * cus); }
  if (!mark(3)) return MOE_ERR_HIP;

  const int n4 = k * (H / 4);
  k_combine<<<(n4 + 255) / 256, 256, 0, s>>>(d.part, x, y, H, L->top_k, k, L->shared_inter > 0,
                                            (flags & MOE_RESIDUAL) ? 1 : 0);
  if (!mark(4)) return MOE_ERR_HIP;
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
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

size_t accept_prefix_workspace_size(int32_t n_target, int32_t vocab) {
  if (n_target < 1 || n_target > 64 || vocab < 1 || vocab > (1 << 24)) return 0;
  const size_t nchunks = ((size_t)vocab + AM_CHUNK - 1) / AM_CHUNK;
  return align256((size_t)n_target * nchunks * 4) * 2;
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
  float* pv = (float*)workspace;
  int* pi = (int*)((uint8_t*)workspace + need / 2);
  hipStream_t s = (hipStream_t)hip_stream;
  (void)hipGetLastError();
  k_argmax_partial<<<dim3(nchunks, n_target), 256, 0, s>>>(logits, vocab, nchunks, pv, pi);
  k_accept_final<<<1, 64, 0, s>>>(pv, pi, nchunks, n_target, draft_ids, n_draft, target_ids, accepted);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
