// The MLP of the BiFormer block in one launch (bf16):
//   out = r + fc2(GELU(fc1(x))),  fc1: C -> Hd, fc2: Hd -> C,
// with the hidden layer rounded once to bf16 (the stored-layer reading of
// the block: every layer output a bf16 tensor) but never written to memory.
//
// Page keys: p1 = cybasar.com "CVPR2023: BiFormer中的双层路由注意力机制解析"
// (§2: a BiFormer block is the BRA attention followed by a 2-layer MLP, each
// with a residual connection).  The block's other layers (position conv,
// LayerNorm, the BRA module) are separate launches.
//
// Work split.  A workgroup owns 4 TW tokens (wavefront w: TW tokens, one or
// two 16-token MFMA column blocks) and walks the hidden layer in chunks of
// 32 features; each chunk's rows of W1 (32 x C), its columns of W2 (C x 32)
// and its 32 biases are staged in LDS (two buffers: the next chunk is loaded
// into registers while the current one is multiplied; one barrier a chunk).
// Per chunk, on each wavefront, with everything in registers:
//   fc1  H^T (32 x TW) = W1_j X^T on v_mfma_f32_16x16x32_bf16, X^T read
//        once per launch straight into the operand layout (a lane holds 8
//        consecutive channels of one token);
//   act  GELU (exact erf form; the fc1 accumulators start at b1), rounded
//        to bf16;
//   fc2  OUT^T (C x TW) += W2_j H^T.  fc1 leaves each lane with hidden rows
//        4lg..4lg+3 of both 16-row halves of the chunk; the k order of fc2
//        is permuted to match (slot 8lg + e holds hidden 4lg + e for e < 4,
//        16 + 4lg + e - 4 above) and W2's columns are staged in that order,
//        so H^T becomes fc2's B operand without moving.
// Epilogue: lanes lg, lg^1 trade fp32 halves of two output tiles
// (v_permlane16_swap), so each holds 8 consecutive channels of one token;
// + b2 + r in fp32, one rounding, 16-byte stores.

#include "device_common.h"

namespace bra {
namespace {

constexpr uint32_t kMlpOob = 0x80000000u;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int C_, int TW_>
struct Mg {
  static constexpr int C = C_, TW = TW_;
  static constexpr int NB = TW / 16;          // 16-token column blocks a wavefront
  static constexpr int KS = C / 32;           // 32-channel k steps of fc1
  static constexpr int OT = C / 16;           // 16-channel output tiles of fc2
  static constexpr int TOK = 4 * TW;          // tokens a workgroup
  static constexpr int W1E = 4 * C;           // 16-byte chunks of one W1 chunk (32 x C)
  static constexpr int W2E = 4 * C;           // 16-byte chunks of one W2 chunk (C x 32)
  static constexpr int N1 = (W1E + kThreads - 1) / kThreads;   // per thread
  static constexpr int N2 = (W2E + kThreads - 1) / kThreads;
  static constexpr int BUF = (32 * C + C * 32) * 2 + 32 * 4;   // W1, W2, b1 of a chunk
  // W1 rows are 2C bytes: 16-byte chunk c of row r sits at c ^ ((r >> SH) & MSK),
  // so the 16 rows one operand read touches fill 16 distinct 16-byte slots
  static constexpr int SH = C == 64 ? 1 : 0, MSK = C == 64 ? 7 : 15;
  static_assert(C == 64 || C == 128 || C == 256, "channels");
  static_assert(TW == 16 || TW == 32, "tokens a wavefront");
};

struct MlpArgs {
  const uint16_t* x;     // [T, C]
  const uint16_t* w1;    // [Hd, C]
  const float* b1;       // [Hd] or null
  const uint16_t* w2;    // [C, Hd]
  const float* b2;       // [C] or null
  const uint16_t* r;     // residual [T, C]
  uint16_t* out;         // [T, C]
  int T, Hd;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mlp_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 mload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 mload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <class G>
__global__ __launch_bounds__(kThreads) void mlp_kernel(MlpArgs A) {
  constexpr int C = G::C, NB = G::NB, KS = G::KS, OT = G::OT, N1 = G::N1, N2 = G::N2;
  constexpr int SH = G::SH, MSK = G::MSK;
  extern __shared__ __align__(16) unsigned char lds[];
  float* b2s = (float*)(lds + 2 * G::BUF);        // [C]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 15, lg = lane >> 4;
  const int T = A.T, Hd = A.Hd;
  const int tok0 = blockIdx.x * G::TOK + wave * G::TW;   // first token of this wavefront
  const uint32_t tbytes = (uint32_t)T * C * 2;
  const auto Xr = mlp_rsrc(A.x, tbytes);
  const auto Rr = mlp_rsrc(A.r, tbytes);
  const auto Or = mlp_rsrc(A.out, tbytes);
  const auto W1r = mlp_rsrc(A.w1, (uint32_t)Hd * C * 2);
  const auto W2r = mlp_rsrc(A.w2, (uint32_t)C * Hd * 2);

  // X^T operands: token tok0 + 16 nb + lq, channels 32 s + 8 lg .. +7
  bf16x8 xo[NB][KS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int t = tok0 + 16 * nb + lq;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t off = t < T ? (uint32_t)(t * C + 32 * s + 8 * lg) * 2 : kMlpOob;
      xo[nb][s] = __builtin_bit_cast(bf16x8, mload16(Xr, off));
    }
  }
  for (int c = tid; c < C; c += kThreads) b2s[c] = A.b2 ? A.b2[c] : 0.f;

  // staging of hidden chunk j: W1 rows j*32 .. j*32+31 (chunk c of row r at
  // c ^ ((r >> SH) & MSK)); W2 columns j*32 .. +31 of every row o, 16-byte
  // chunk g holding hidden 4g..4g+3 and 16+4g..16+4g+3 of the chunk (the
  // permuted k order of fc2), at g ^ ((o >> 2) & 3); b1 of the chunk
  uint4 p1[N1];
  uint2 p2a[N2], p2b[N2];
  float pb1 = 0.f;
  auto prefetch = [&](int j) {
#pragma unroll
    for (int i = 0; i < N1; ++i) {
      const int e = i * kThreads + tid;
      const int r = e / (C / 8), c = e % (C / 8);
      p1[i] = mload16(W1r, e < G::W1E ? (uint32_t)((j * 32 + r) * C + 8 * c) * 2 : kMlpOob);
    }
#pragma unroll
    for (int i = 0; i < N2; ++i) {
      const int e = i * kThreads + tid;
      const int o = e >> 2, g = e & 3;
      const uint32_t base = (uint32_t)(o * Hd + j * 32 + 4 * g) * 2;
      p2a[i] = mload8(W2r, e < G::W2E ? base : kMlpOob);
      p2b[i] = mload8(W2r, e < G::W2E ? base + 32 : kMlpOob);
    }
    if (tid < 32) pb1 = A.b1 ? A.b1[j * 32 + tid] : 0.f;
  };
  auto commit = [&](int buf) {
    unsigned char* bp = lds + buf * G::BUF;
    uint16_t* W1s = (uint16_t*)bp;
    uint16_t* W2s = W1s + 32 * C;
    float* b1s = (float*)(bp + (32 * C + C * 32) * 2);
#pragma unroll
    for (int i = 0; i < N1; ++i) {
      const int e = i * kThreads + tid;
      if (e < G::W1E) {
        const int r = e / (C / 8), c = e % (C / 8);
        *(uint4*)(W1s + r * C + ((c ^ ((r >> SH) & MSK)) << 3)) = p1[i];
      }
    }
#pragma unroll
    for (int i = 0; i < N2; ++i) {
      const int e = i * kThreads + tid;
      if (e < G::W2E) {
        const int o = e >> 2, g = e & 3;
        *(uint4*)(W2s + o * 32 + ((g ^ ((o >> 2) & 3)) << 3)) =
            make_uint4(p2a[i].x, p2a[i].y, p2b[i].x, p2b[i].y);
      }
    }
    if (tid < 32) b1s[tid] = pb1;
  };

  f32x4 acc[NB][OT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int o = 0; o < OT; ++o) acc[nb][o] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nch = Hd / 32;
  prefetch(0);
  commit(0);
  __syncthreads();
  for (int j = 0; j < nch; ++j) {
    if (j + 1 < nch) prefetch(j + 1);
    const unsigned char* bp = lds + (j & 1) * G::BUF;
    const uint16_t* W1s = (const uint16_t*)bp;
    const uint16_t* W2s = W1s + 32 * C;
    const float* b1s = (const float*)(bp + (32 * C + C * 32) * 2);

    // ---- fc1: H^T rows 16t + 4lg + e of this lane's token columns, the
    // accumulators starting at b1 ----
    const float4 bA = *(const float4*)(b1s + 4 * lg);
    const float4 bB = *(const float4*)(b1s + 16 + 4 * lg);
    f32x4 h[2][NB];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float4 bt = t ? bB : bA;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) h[t][nb] = f32x4{bt.x, bt.y, bt.z, bt.w};
      const int row = 16 * t + lq;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int c = 4 * s + lg;
        const bf16x8 a =
            *(const bf16x8*)(W1s + row * C + ((c ^ ((row >> SH) & MSK)) << 3));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) h[t][nb] = mfma16(a, xo[nb][s], h[t][nb]);
      }
    }
    // ---- GELU, one rounding; fc2's B operand in the permuted k order ----
    bf16x8 hop[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t u0 = pack_bf16x2(gelu_as(h[0][nb][0]), gelu_as(h[0][nb][1]));
      const uint32_t u1 = pack_bf16x2(gelu_as(h[0][nb][2]), gelu_as(h[0][nb][3]));
      const uint32_t u2 = pack_bf16x2(gelu_as(h[1][nb][0]), gelu_as(h[1][nb][1]));
      const uint32_t u3 = pack_bf16x2(gelu_as(h[1][nb][2]), gelu_as(h[1][nb][3]));
      hop[nb] = __builtin_bit_cast(bf16x8, make_uint4(u0, u1, u2, u3));
    }
    // ---- fc2: OUT^T rows 16o + 4lg + e += W2_j H^T ----
#pragma unroll
    for (int o = 0; o < OT; ++o) {
      const int row = 16 * o + lq;
      const bf16x8 a = *(const bf16x8*)(W2s + row * 32 + ((lg ^ ((row >> 2) & 3)) << 3));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb][o] = mfma16(a, hop[nb], acc[nb][o]);
    }
    // the other buffer was last read before the previous barrier
    if (j + 1 < nch) commit((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: lanes lg, lg^1 trade halves of output tiles 2m, 2m+1 ----
  const bool odd = lg & 1;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int t = tok0 + 16 * nb + lq;
#pragma unroll
    for (int m = 0; m < OT / 2; ++m) {
      const f32x4 f0 = acc[nb][2 * m], f1 = acc[nb][2 * m + 1];
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(f0[e]),
                                                         __float_as_uint(f1[e]), false, false);
        // even rows: channels 4lg .. 4lg+7 of the pair; odd rows: 16 + 4(lg-1) .. +7
        if (odd) {
          v[e] = __uint_as_float(sw[0]);
          v[4 + e] = f1[e];
        } else {
          v[e] = f0[e];
          v[4 + e] = __uint_as_float(sw[1]);
        }
      }
      const int ch = 32 * m + (odd ? 16 + 4 * (lg - 1) : 4 * lg);
      const uint32_t off = t < T ? (uint32_t)(t * C + ch) * 2 : kMlpOob;
      const uint4 rv = mload16(Rr, off);
      const uint32_t ru[4] = {rv.x, rv.y, rv.z, rv.w};
      uint32_t ov[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a0 = v[2 * q] + b2s[ch + 2 * q] + bf16_lo(ru[q]);
        const float a1 = v[2 * q + 1] + b2s[ch + 2 * q + 1] + bf16_hi(ru[q]);
        ov[q] = pack_bf16x2(a0, a1);
      }
      const u32x4 x = {ov[0], ov[1], ov[2], ov[3]};
      __builtin_amdgcn_raw_buffer_store_b128(x, Or, off, 0, 0);
    }
  }
}

template <class G>
hipError_t mlp_launch(const MlpArgs& a, hipStream_t st) {
  const size_t lds = 2 * (size_t)G::BUF + (size_t)G::C * 4;
  const void* fn = reinterpret_cast<const void*>(&mlp_kernel<G>);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const long long groups = ((long long)a.T + G::TOK - 1) / G::TOK;
  hipLaunchKernelGGL(mlp_kernel<G>, dim3((unsigned)groups), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mlp(const void* x, long long T, int C, int Hd, const void* w1, const float* b1,
                      const void* w2, const float* b2, const void* resid, void* out,
                      hipStream_t st) {
  if (T <= 0 || Hd <= 0 || Hd % 32) return hipErrorNotSupported;
  if (C != 64 && C != 128 && C != 256) return hipErrorNotSupported;
  // buffer offsets are 32-bit
  if (T * C * 2 >= (long long)kMlpOob || (long long)Hd * C * 2 >= (long long)kMlpOob)
    return hipErrorNotSupported;
  MlpArgs a;
  a.x = (const uint16_t*)x; a.w1 = (const uint16_t*)w1; a.b1 = b1;
  a.w2 = (const uint16_t*)w2; a.b2 = b2; a.r = (const uint16_t*)resid; a.out = (uint16_t*)out;
  a.T = (int)T; a.Hd = Hd;
  if (C == 64) return mlp_launch<Mg<64, 32>>(a, st);
  if (C == 128) return mlp_launch<Mg<128, 16>>(a, st);
  return mlp_launch<Mg<256, 16>>(a, st);
}

}  // namespace bra
