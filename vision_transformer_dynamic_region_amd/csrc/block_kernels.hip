// Kernels of the BiFormer block around the BRA module (gfx950): the residual
// 3x3 depthwise position-encoding conv and LayerNorm.
//
// Page keys: p1 = cybasar.com "CVPR2023: BiFormer中的双层路由注意力机制解析"
// (§4: a 3x3 convolution encodes position implicitly; a two-layer MLP of
// ratio 3), p3 = the BiFormer architecture page (§3.1: pre-norm blocks,
// x + bra(norm1(x)), x + ffn(norm2(x)), nn.LayerNorm).

#include "device_common.h"

namespace bra {
namespace {

// out = x + b + depthwise 3x3 cross-correlation of x (zero padding 1), one
// rounding.  A thread owns one 16-byte channel group of one pixel and reads
// the 9 neighbouring vectors (the tile's pixels are shared through L1/L2);
// consecutive threads take consecutive groups of a pixel, then pixels along
// a row, so every load and the store are coalesced.
struct PosArgs {
  const void* x;
  const float* w;       // [C, 3, 3]
  const float* b;       // [C] or null
  void* out;
  int H, W, C, G;       // G = 16-byte groups per pixel
  long long total;      // B * H * W * G
};

template <bool BF16>
__global__ __launch_bounds__(kThreads) void pos_conv_kernel(PosArgs a) {
  constexpr int VEC = BF16 ? 8 : 4;
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= a.total) return;
  const int g = (int)(i % a.G);
  const long long p = i / a.G;                      // pixel index b*H*W + y*W + x
  const int xq = (int)(p % a.W);
  const long long by = p / a.W;
  const int yq = (int)(by % a.H);
  const uint4* X = (const uint4*)a.x;
  float acc[VEC], ctr[VEC];
  unpack16<BF16>(X[i], ctr);
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = ctr[e] + (a.b ? a.b[g * VEC + e] : 0.f);
#pragma unroll
  for (int dy = -1; dy <= 1; ++dy) {
    if ((unsigned)(yq + dy) >= (unsigned)a.H) continue;
#pragma unroll
    for (int dx = -1; dx <= 1; ++dx) {
      if ((unsigned)(xq + dx) >= (unsigned)a.W) continue;
      float v[VEC];
      unpack16<BF16>(X[i + ((long long)dy * a.W + dx) * a.G], v);
      const int tap = (dy + 1) * 3 + (dx + 1);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = fmaf(a.w[(g * VEC + e) * 9 + tap], v[e], acc[e]);
    }
  }
  uint4 o;
  if constexpr (BF16) {
    o = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  } else {
    o = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                   __float_as_uint(acc[3]));
  }
  ((uint4*)a.out)[i] = o;
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
                           bool bf16, void* out, hipStream_t st) {
  PosArgs a;
  a.x = x; a.w = w; a.b = b; a.out = out;
  a.H = s.H; a.W = s.W; a.C = s.C;
  a.G = s.C / (bf16 ? 8 : 4);
  a.total = (long long)s.B * s.H * s.W * a.G;
  const dim3 grid((unsigned)((a.total + kThreads - 1) / kThreads));
  if (bf16)
    hipLaunchKernelGGL(pos_conv_kernel<true>, grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(pos_conv_kernel<false>, grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

// Lanes per row and groups per lane for a LayerNorm over C channels, or
// false when a lane would need more than 4 groups.
bool layer_norm_shape(int C, bool bf16, int* L, int* NG) {
  const int vec = bf16 ? 8 : 4;
  if (C % vec) return false;
  const int G = C / vec;
  int l = 1;
  while (l * 2 <= 64 && G % (l * 2) == 0) l *= 2;
  if (G / l > 4) return false;
  *L = l;
  *NG = G / l;
  return true;
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
