// Kernels of the BiFormer block around the BRA module (gfx950): the residual
// 3x3 depthwise position-encoding conv and LayerNorm.
//
// Page keys: p1 = cybasar.com "CVPR2023: BiFormer中的双层路由注意力机制解析"
// (§4: a 3x3 convolution encodes position implicitly; a two-layer MLP of
// ratio 3), p3 = the BiFormer architecture page (§3.1: pre-norm blocks,
// x + bra(norm1(x)), x + ffn(norm2(x)), nn.LayerNorm).

#include "device_common.h"

#include <type_traits>

namespace bra {
namespace {

// out = x + b + depthwise 3x3 cross-correlation of x (zero padding 1), one
// rounding.  Thread (x, g) owns 16-byte channel group g of pixel column x
// over a strip of sr rows: its 9 x VEC weights are loaded once, and a
// circular window of three rows of three vectors walks down the strip.  The
// rows come in batches of three, loaded together by buffer loads that read
// zero outside the image (no branches); within a batch the window's slots are
// compile-time, so no data moves.  Consecutive threads take consecutive
// groups of a pixel, then pixels along the row, so every load and the store
// are coalesced.  32-bit offsets within an image.
// Strips are whole batches of three rows, at least kPosMinRows long, and
// the shortest such that the launch is at most one generation of resident
// wavefronts: kPosWaves = 1024 SIMDs x the 2 a SIMD holds at this kernel's
// register use (190 VGPRs).  A second generation pays the window prologue
// and the first batch's wait again (on MI355X the 64-image 56 x 56 x 64 shape
// took 23.0 us with 9-row strips, 19.5 with 15).
constexpr int kPosMinRows = 9;
constexpr long long kPosWaves = 2048;

struct PosArgs {
  const void* x;
  const float* w;       // [C, 3, 3]
  const float* b;       // [C] or null
  void* out;
  // LN: out's LayerNorm as well (gamma lng, beta lnb, eps) into nout
  const float* lng;
  const float* lnb;
  float eps;
  void* nout;
  int H, W, C, G;       // G = 16-byte groups per pixel
  int row_items;        // W * G
  int sr;               // rows a strip (a multiple of 3)
  FastDiv f_G;
};

typedef uint32_t pos_u32x4 __attribute__((ext_vector_type(4)));

// Sum over aligned groups of GL consecutive lanes: DPP lane moves within
// rows of 16 (xor 1, xor 2, then the mirrored half of 8 and of 16, each
// pairing every lane with one of the other half), lane swaps across rows.
template <int GL>
__device__ __forceinline__ float lane_group_sum(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), decltype(ctrl)::value, 0xf, 0xf, false));
  };
  if constexpr (GL > 1) v += dpp(v, std::integral_constant<int, 0xB1>());   // quad_perm 1,0,3,2
  if constexpr (GL > 2) v += dpp(v, std::integral_constant<int, 0x4E>());   // quad_perm 2,3,0,1
  if constexpr (GL > 4) v += dpp(v, std::integral_constant<int, 0x141>());  // row_half_mirror
  if constexpr (GL > 8) v += dpp(v, std::integral_constant<int, 0x140>());  // row_mirror
  if constexpr (GL > 16) v += xor16(v);
  if constexpr (GL > 32) v += xor32(v);
  return v;
}

// With GL > 0 (LN), the LayerNorm of each output pixel too (the block's LN1
// of x1): a pixel's G = GL groups are GL consecutive lanes, so its float32
// statistics of the rounded x1 (mean, then the biased variance around it,
// as layer_norm_kernel) are lane sums; one rounding.
template <bool BF16, int GL>
__global__ __launch_bounds__(kThreads) void pos_conv_kernel(PosArgs a) {
  constexpr bool LN = GL > 0;
  constexpr int VEC = BF16 ? 8 : 4;
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= a.row_items) return;
  const int y0 = blockIdx.y * a.sr, b = blockIdx.z;
  const int xq = fdiv(t, a.f_G), g = t - xq * a.G;
  const uint32_t img_bytes = (uint32_t)a.H * a.row_items * 16;
  const auto X = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>((const void*)((const uint4*)a.x + (size_t)b * a.H * a.row_items)), (short)0,
      (int)img_bytes, 0x00020000);
  uint4* O = (uint4*)a.out + (size_t)b * a.H * a.row_items;
  uint4* NO = LN ? (uint4*)a.nout + (size_t)b * a.H * a.row_items : nullptr;
  float wt[VEC][9], bias[VEC], lg_[VEC], lb_[VEC];
  {
    const float4* wp = (const float4*)(a.w + g * VEC * 9);   // VEC * 9 contiguous floats
#pragma unroll
    for (int k = 0; k < VEC * 9 / 4; ++k) {
      const float4 f = wp[k];
      const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) wt[(4 * k + u) / 9][(4 * k + u) % 9] = fv[u];
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) bias[e] = a.b ? a.b[g * VEC + e] : 0.f;
    if constexpr (LN) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        lg_[e] = a.lng[g * VEC + e];
        lb_[e] = a.lnb[g * VEC + e];
      }
    }
  }
  const bool colok[3] = {xq > 0, true, xq + 1 < a.W};
  // vector at (y, x + c - 1), zero outside the image
  auto ld = [&](int y, int c) -> uint4 {
    const uint32_t off = ((unsigned)y < (unsigned)a.H && colok[c])
                             ? (uint32_t)(y * a.row_items + t + (c - 1) * a.G) * 16 : 0x80000000u;
    const pos_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(X, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
  };
  // while row y = yb + u of a batch is computed, row y - 1 + r sits in slot
  // (u + r) % 3
  uint4 win[3][3];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 3; ++c) win[r][c] = ld(y0 - 1 + r, c);
  const int y1 = min(y0 + a.sr, a.H);
  for (int yb = y0; yb < y1; yb += 3) {
    uint4 nx[3][3];
#pragma unroll
    for (int u = 0; u < 3; ++u)
#pragma unroll
      for (int c = 0; c < 3; ++c) nx[u][c] = ld(yb + u + 1, c);
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int y = yb + u;
#pragma unroll
      for (int c = 0; c < 3; ++c) win[(u + 2) % 3][c] = nx[u][c];
      float acc[VEC], v[VEC];
      unpack16<BF16>(win[(u + 1) % 3][1], v);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = v[e] + bias[e];
#pragma unroll
      for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int c = 0; c < 3; ++c) {
          unpack16<BF16>(win[(u + r) % 3][c], v);
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[e] = fmaf(wt[e][r * 3 + c], v[e], acc[e]);
        }
      uint4 o;
      if constexpr (BF16) {
        o = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                       pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
      } else {
        o = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                       __float_as_uint(acc[3]));
      }
      if (y < y1) O[y * a.row_items + t] = o;
      if constexpr (LN) {
        float xr[VEC];
        if constexpr (BF16) {
          unpack16<true>(o, xr);
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) xr[e] = acc[e];
        }
        float sm = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) sm += xr[e];
        sm = lane_group_sum<GL>(sm);
        const float mean = sm / (float)a.C;
        float q = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float d = xr[e] - mean;
          q = fmaf(d, d, q);
        }
        q = lane_group_sum<GL>(q);
        const float rstd = 1.0f / sqrtf(q / (float)a.C + a.eps);
        float nv[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) nv[e] = (xr[e] - mean) * rstd * lg_[e] + lb_[e];
        uint4 n;
        if constexpr (BF16) {
          n = make_uint4(pack_bf16x2(nv[0], nv[1]), pack_bf16x2(nv[2], nv[3]),
                         pack_bf16x2(nv[4], nv[5]), pack_bf16x2(nv[6], nv[7]));
        } else {
          n = make_uint4(__float_as_uint(nv[0]), __float_as_uint(nv[1]), __float_as_uint(nv[2]),
                         __float_as_uint(nv[3]));
        }
        if (y < y1) NO[y * a.row_items + t] = n;
      }
    }
  }
}

// LayerNorm over the C channels of each row (p3 §3.1 nn.LayerNorm): float32
// mean, then the biased variance around it, y = (x - mean) * rsqrt(var +
// eps) * g + b, one rounding.  L lanes share a row (L a power of two
// dividing the row's 16-byte groups, at most 64), each holding NG groups in
// registers; the sums are reduced across the L lanes with xor shuffles.
struct NormArgs {
  const void* x;
  const float* g;
  const float* b;
  void* y;
  long long rows;
  int C, G, L;          // groups per row, lanes per row
  float eps;
};

template <bool BF16, int NG>
__global__ __launch_bounds__(kThreads) void layer_norm_kernel(NormArgs a) {
  constexpr int VEC = BF16 ? 8 : 4;
  const int lane = threadIdx.x & 63;
  const int rpw = 64 / a.L;                         // rows per wavefront
  const long long row = ((long long)blockIdx.x * kWaves + (threadIdx.x >> 6)) * rpw + lane / a.L;
  const int li = lane % a.L;
  const bool ok = row < a.rows;                     // lanes past the end still shuffle
  const uint4* X = (const uint4*)a.x + (ok ? row : 0) * a.G;
  float v[NG][VEC];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    unpack16<BF16>(X[li + j * a.L], v[j]);
#pragma unroll
    for (int e = 0; e < VEC; ++e) s += v[j][e];
  }
  for (int m = 1; m < a.L; m <<= 1) s += __shfl_xor(s, m, 64);
  const float mean = s / (float)a.C;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < NG; ++j)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float d = v[j][e] - mean;
      q = fmaf(d, d, q);
    }
  for (int m = 1; m < a.L; m <<= 1) q += __shfl_xor(q, m, 64);
  const float rstd = 1.0f / sqrtf(q / (float)a.C + a.eps);
  if (!ok) return;
  uint4* Y = (uint4*)a.y + row * a.G;
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int c0 = (li + j * a.L) * VEC;
    float o[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] = (v[j][e] - mean) * rstd * a.g[c0 + e] + a.b[c0 + e];
    if constexpr (BF16) {
      Y[li + j * a.L] = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                   pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
    } else {
      Y[li + j * a.L] = make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]),
                                   __float_as_uint(o[2]), __float_as_uint(o[3]));
    }
  }
}

}  // namespace

hipError_t launch_pos_conv(const void* x, const float* w, const float* b, const Shape& s,
                           bool bf16, void* out, hipStream_t st, const float* ln_g,
                           const float* ln_b, float eps, void* nout) {
  PosArgs a;
  a.x = x; a.w = w; a.b = b; a.out = out;
  a.lng = ln_g; a.lnb = ln_b; a.eps = eps; a.nout = nout;
  a.H = s.H; a.W = s.W; a.C = s.C;
  a.G = s.C / (bf16 ? 8 : 4);
  a.row_items = s.W * a.G;
  a.f_G = make_fastdiv(a.G);
  if (s.H > 65535 || s.B > 65535) return hipErrorInvalidValue;
  // byte offsets within an image stay below the out-of-range marker
  if ((long long)s.H * a.row_items * 16 >= 0x80000000LL) return hipErrorInvalidValue;
  const long long per_strip = (long long)((a.row_items + kThreads - 1) / kThreads) * s.B * kWaves;
  a.sr = kPosMinRows;
  while (a.sr < s.H && per_strip * ((s.H + a.sr - 1) / a.sr) > kPosWaves) a.sr += 3;
  const dim3 grid((unsigned)((a.row_items + kThreads - 1) / kThreads),
                  (unsigned)((s.H + a.sr - 1) / a.sr), (unsigned)s.B);
  if (nout) {
    // a pixel's groups share one 64-lane wavefront: G a power of two, 4..64
    if (!ln_g || !ln_b) return hipErrorNotSupported;
#define BRA_POS_LN(GG)                                                              \
    if (a.G == GG) {                                                                \
      if (bf16)                                                                     \
        hipLaunchKernelGGL((pos_conv_kernel<true, GG>), grid, dim3(kThreads), 0, st, a);  \
      else                                                                          \
        hipLaunchKernelGGL((pos_conv_kernel<false, GG>), grid, dim3(kThreads), 0, st, a); \
      return hipGetLastError();                                                     \
    }
    BRA_POS_LN(4) BRA_POS_LN(8) BRA_POS_LN(16) BRA_POS_LN(32) BRA_POS_LN(64)
#undef BRA_POS_LN
    return hipErrorNotSupported;
  }
  if (bf16)
    hipLaunchKernelGGL((pos_conv_kernel<true, 0>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((pos_conv_kernel<false, 0>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_layer_norm(const void* x, long long rows, int C, const float* g,
                             const float* b, float eps, bool bf16, void* y, hipStream_t st) {
  NormArgs a;
  int L = 0, NG = 0;
  if (rows <= 0 || !layer_norm_shape(C, bf16, &L, &NG)) return hipErrorInvalidValue;
  a.x = x; a.g = g; a.b = b; a.y = y; a.rows = rows; a.C = C;
  a.G = C / (bf16 ? 8 : 4);
  a.L = L;
  a.eps = eps;
  const long long per_block = (long long)kWaves * (64 / L);
  const dim3 grid((unsigned)((rows + per_block - 1) / per_block));
#define BRA_LN(BB, NN) hipLaunchKernelGGL((layer_norm_kernel<BB, NN>), grid, dim3(kThreads), 0, st, a)
  switch (NG) {
    case 1: if (bf16) BRA_LN(true, 1); else BRA_LN(false, 1); break;
    case 2: if (bf16) BRA_LN(true, 2); else BRA_LN(false, 2); break;
    case 3: if (bf16) BRA_LN(true, 3); else BRA_LN(false, 3); break;
    default: if (bf16) BRA_LN(true, 4); else BRA_LN(false, 4); break;
  }
#undef BRA_LN
  return hipGetLastError();
}

}  // namespace bra
