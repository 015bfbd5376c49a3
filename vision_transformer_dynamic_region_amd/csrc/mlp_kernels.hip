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
// Epilogue: + b2 + r in fp32 in the MFMA layout (a lane holds channels
// 16o + 4lg .. +3 of one token for each 16-channel tile o); lanes lg, lg^1
// then trade halves of two tiles (v_permlane16_swap), so each holds 8
// consecutive channels; one rounding, 16-byte stores.
//
// Block-tail form (TAIL): the block's last three layers in the same launch,
//   x2 = x1 + y W_out^T + b_out,  n2 = LN2(x2),  out = x2 + MLP(n2),
// x2 and n2 rounded to bf16 as the block stores them (and written to the
// block's workspace), with y the BRA module's attention output.  W_out is
// staged in LDS; the output projection on the MFMAs leaves a lane with 4C/16
// channels of one token (tiles o, rows 4lg..4lg+3), so LN2's statistics are
// a lane sum and two lane swaps, and n2 becomes fc1's B operand directly:
// fc1's k order is permuted as fc2's is (slot 8lg + e of k step s holds
// channel 32s + 4lg + e for e < 4, 32s + 16 + 4lg + e - 4 above) and W1's
// columns are staged in that order.  x2 stays in registers as the MLP's
// residual.

#include "device_common.h"

namespace bra {
namespace {

constexpr uint32_t kMlpOob = 0x80000000u;
#ifndef BRA_TAIL_TW64
#define BRA_TAIL_TW64 16
#endif
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
  const uint16_t* x;     // [T, C]: the MLP's input (TAIL: y, the attention output)
  const uint16_t* w1;    // [Hd, C]
  const float* b1;       // [Hd] or null
  const uint16_t* w2;    // [C, Hd]
  const float* b2;       // [C] or null
  const uint16_t* r;     // residual [T, C] (TAIL: x1, the output projection's)
  uint16_t* out;         // [T, C]
  // TAIL only
  const uint16_t* wo;    // [C, C] output projection
  const float* bo;       // [C] or null
  const float* lng;      // [C] LN2 gamma
  const float* lnb;      // [C] LN2 beta
  float eps;
  uint16_t* x2;          // [T, C] or null: x2 stored
  uint16_t* n2;          // [T, C] or null: LN2(x2) stored
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

// LDS layout: two chunk buffers [W1 32 x C | W2 C x 32 | b1 32], then b2
// [C]; TAIL adds b_out, gamma, beta [C] each and W_out [C x C].
template <class G, bool TAIL>
struct MlpLds {
  static constexpr int C = G::C;
  static constexpr int B2 = 2 * G::BUF;
  static constexpr int BO = B2 + C * 4;
  static constexpr int LG = BO + C * 4;
  static constexpr int LB = LG + C * 4;
  static constexpr int WO = LB + C * 4;
  static constexpr int BYTES = TAIL ? WO + C * C * 2 : BO;
};

template <class G, bool TAIL>
__global__ __launch_bounds__(kThreads) void mlp_kernel(MlpArgs A) {
  constexpr int C = G::C, NB = G::NB, KS = G::KS, OT = G::OT, N1 = G::N1, N2 = G::N2;
  constexpr int SH = G::SH, MSK = G::MSK;
  using L = MlpLds<G, TAIL>;
  extern __shared__ __align__(16) unsigned char lds[];
  float* b2s = (float*)(lds + L::B2);              // [C]

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
  // this lane's token of column block nb, and the byte offset of its
  // channels 16o + 4lg .. +3 (the MFMA output layout)
  auto tok = [&](int nb) { return tok0 + 16 * nb + lq; };
  auto moff = [&](int nb, int o) -> uint32_t {
    return tok(nb) < T ? (uint32_t)(tok(nb) * C + 16 * o + 4 * lg) * 2 : kMlpOob;
  };

  // the input's operands in natural channel order: lane (lq, lg) holds
  // channels 32 s + 8 lg .. +7 of token tok(nb)
  bf16x8 xo[NB][KS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t off = tok(nb) < T ? (uint32_t)(tok(nb) * C + 32 * s + 8 * lg) * 2 : kMlpOob;
      xo[nb][s] = __builtin_bit_cast(bf16x8, mload16(Xr, off));
    }
  // the residual of the MLP in the MFMA output layout, as bf16 pairs (TAIL:
  // x2, computed below; else loaded for the epilogue)
  uint2 res[NB][OT];
  for (int c = tid; c < C; c += kThreads) b2s[c] = A.b2 ? A.b2[c] : 0.f;

  if constexpr (TAIL) {
    // ---- x2 = x1 + y W_out^T + b_out, rounded; n2 = LN2(x2), rounded ----
    float* bos = (float*)(lds + L::BO);
    float* lgs = (float*)(lds + L::LG);
    float* lbs = (float*)(lds + L::LB);
    uint16_t* Wos = (uint16_t*)(lds + L::WO);
    const auto Wor = mlp_rsrc(A.wo, (uint32_t)C * C * 2);
    for (int e = tid; e < C * C / 8; e += kThreads) {
      const int r = e / (C / 8), c = e % (C / 8);
      *(uint4*)(Wos + r * C + ((c ^ ((r >> SH) & MSK)) << 3)) = mload16(Wor, (uint32_t)e * 16);
    }
    for (int c = tid; c < C; c += kThreads) {
      bos[c] = A.bo ? A.bo[c] : 0.f;
      lgs[c] = A.lng[c];
      lbs[c] = A.lnb[c];
    }
    uint2 x1v[NB][OT];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int o = 0; o < OT; ++o) x1v[nb][o] = mload8(Rr, moff(nb, o));
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float v[OT][4];
#pragma unroll
      for (int o = 0; o < OT; ++o) {
        const float4 bo4 = *(const float4*)(bos + 16 * o + 4 * lg);
        f32x4 a = {bo4.x, bo4.y, bo4.z, bo4.w};
        const int row = 16 * o + lq;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const int c = 4 * s + lg;
          const bf16x8 w = *(const bf16x8*)(Wos + row * C + ((c ^ ((row >> SH) & MSK)) << 3));
          a = mfma16(w, xo[nb][s], a);
        }
        // + x1, one rounding: the stored x2
        const uint32_t p0 = pack_bf16x2(a[0] + bf16_lo(x1v[nb][o].x), a[1] + bf16_hi(x1v[nb][o].x));
        const uint32_t p1 = pack_bf16x2(a[2] + bf16_lo(x1v[nb][o].y), a[3] + bf16_hi(x1v[nb][o].y));
        res[nb][o] = make_uint2(p0, p1);
        v[o][0] = bf16_lo(p0); v[o][1] = bf16_hi(p0);
        v[o][2] = bf16_lo(p1); v[o][3] = bf16_hi(p1);
        if (A.x2) {
          const u32x2 st = {p0, p1};
          __builtin_amdgcn_raw_buffer_store_b64(st, mlp_rsrc(A.x2, tbytes), moff(nb, o), 0, 0);
        }
      }
      // LN2 over the token's C channels: 4C/16 a lane, the 4 lanes of one
      // token (lg) combined by two lane swaps; float32, two passes
      float sm = 0.f;
#pragma unroll
      for (int o = 0; o < OT; ++o) sm += (v[o][0] + v[o][1]) + (v[o][2] + v[o][3]);
      sm += xor16(sm);
      sm += xor32(sm);
      const float mean = sm / (float)C;
      float sq = 0.f;
#pragma unroll
      for (int o = 0; o < OT; ++o)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float d = v[o][e] - mean;
          sq = fmaf(d, d, sq);
        }
      sq += xor16(sq);
      sq += xor32(sq);
      const float rstd = 1.0f / sqrtf(sq / (float)C + A.eps);
      uint32_t np[OT][2];
#pragma unroll
      for (int o = 0; o < OT; ++o) {
        const float4 g4 = *(const float4*)(lgs + 16 * o + 4 * lg);
        const float4 b4 = *(const float4*)(lbs + 16 * o + 4 * lg);
        np[o][0] = pack_bf16x2((v[o][0] - mean) * rstd * g4.x + b4.x,
                               (v[o][1] - mean) * rstd * g4.y + b4.y);
        np[o][1] = pack_bf16x2((v[o][2] - mean) * rstd * g4.z + b4.z,
                               (v[o][3] - mean) * rstd * g4.w + b4.w);
        if (A.n2) {
          const u32x2 st = {np[o][0], np[o][1]};
          __builtin_amdgcn_raw_buffer_store_b64(st, mlp_rsrc(A.n2, tbytes), moff(nb, o), 0, 0);
        }
      }
      // fc1's B operands in the permuted k order: step s takes tiles 2s, 2s+1
#pragma unroll
      for (int s = 0; s < KS; ++s)
        xo[nb][s] = __builtin_bit_cast(
            bf16x8, make_uint4(np[2 * s][0], np[2 * s][1], np[2 * s + 1][0], np[2 * s + 1][1]));
    }
  }

  // staging of hidden chunk j: W1 rows j*32 .. j*32+31, 16-byte chunk c of
  // row r at c ^ ((r >> SH) & MSK), holding columns 8c .. 8c+7 (TAIL: columns
  // 32s + 4g .. +3 and 32s + 16 + 4g .. +3 for c = 4s + g, fc1's permuted k
  // order); W2 columns j*32 .. +31 of every row o, 16-byte chunk g holding
  // hidden 4g..4g+3 and 16+4g..16+4g+3 of the chunk (fc2's permuted k
  // order), at g ^ ((o >> 2) & 3); b1 of the chunk
  uint2 p1a[N1], p1b[N1];
  uint2 p2a[N2], p2b[N2];
  float pb1 = 0.f;
  auto prefetch = [&](int j) {
#pragma unroll
    for (int i = 0; i < N1; ++i) {
      const int e = i * kThreads + tid;
      const int r = e / (C / 8), c = e % (C / 8);
      const int ca = TAIL ? 32 * (c >> 2) + 4 * (c & 3) : 8 * c;
      const int cb = TAIL ? ca + 16 : ca + 4;
      const uint32_t row = (uint32_t)(j * 32 + r) * C;
      p1a[i] = mload8(W1r, e < G::W1E ? (row + ca) * 2 : kMlpOob);
      p1b[i] = mload8(W1r, e < G::W1E ? (row + cb) * 2 : kMlpOob);
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
        *(uint4*)(W1s + r * C + ((c ^ ((r >> SH) & MSK)) << 3)) =
            make_uint4(p1a[i].x, p1a[i].y, p1b[i].x, p1b[i].y);
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

  // ---- epilogue: + b2 + residual in the MFMA layout, then lanes lg, lg^1
  // trade halves of output tiles 2m, 2m+1 ----
  if constexpr (!TAIL) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int o = 0; o < OT; ++o) res[nb][o] = mload8(Rr, moff(nb, o));
  }
  const bool odd = lg & 1;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int m = 0; m < OT / 2; ++m) {
      float f[2][4];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int o = 2 * m + q;
        const float4 b4 = *(const float4*)(b2s + 16 * o + 4 * lg);
        f[q][0] = acc[nb][o][0] + b4.x + bf16_lo(res[nb][o].x);
        f[q][1] = acc[nb][o][1] + b4.y + bf16_hi(res[nb][o].x);
        f[q][2] = acc[nb][o][2] + b4.z + bf16_lo(res[nb][o].y);
        f[q][3] = acc[nb][o][3] + b4.w + bf16_hi(res[nb][o].y);
      }
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(f[0][e]),
                                                         __float_as_uint(f[1][e]), false, false);
        // even rows: channels 4lg .. 4lg+7 of the pair; odd rows: 16 + 4(lg-1) .. +7
        if (odd) {
          v[e] = __uint_as_float(sw[0]);
          v[4 + e] = f[1][e];
        } else {
          v[e] = f[0][e];
          v[4 + e] = __uint_as_float(sw[1]);
        }
      }
      const int ch = 32 * m + (odd ? 16 + 4 * (lg - 1) : 4 * lg);
      const uint32_t off = tok(nb) < T ? (uint32_t)(tok(nb) * C + ch) * 2 : kMlpOob;
      const u32x4 x = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                       pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
      __builtin_amdgcn_raw_buffer_store_b128(x, Or, off, 0, 0);
    }
  }
}

template <class G, bool TAIL>
hipError_t mlp_launch(const MlpArgs& a, hipStream_t st) {
  const size_t lds = MlpLds<G, TAIL>::BYTES;
  const void* fn = reinterpret_cast<const void*>(&mlp_kernel<G, TAIL>);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const long long groups = ((long long)a.T + G::TOK - 1) / G::TOK;
  hipLaunchKernelGGL((mlp_kernel<G, TAIL>), dim3((unsigned)groups), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weights-stationary form for C = 64 (Hd <= 256): every chunk of W1, W2 and
// b1 (and in TAIL form W_out) stays in LDS for the whole launch, laid out as
// the chunk buffers above.  Two workgroups of 8 wavefronts a CU; each
// workgroup owns a contiguous range of 16-token blocks and its wavefronts
// claim blocks from an LDS counter, so no barrier follows the staging and
// the blocks of a workgroup are shared out as its wavefronts finish.  A
// wavefront loads the inputs of its next block while it computes the
// current one.
// ---------------------------------------------------------------------------
constexpr int kWsWaves = 8;
constexpr int kWsThreads = kWsWaves * 64;
constexpr int kWsC = 64;
constexpr int kWsChunk = (32 * kWsC + kWsC * 32) * 2 + 32 * 4;   // W1, W2, b1 of a chunk

struct WsLayout {
  int b2, bo, lg, lb, wo, ctr, bytes;
};
__host__ __device__ inline WsLayout ws_layout(int nch, bool tail) {
  WsLayout l;
  int off = nch * kWsChunk;
  l.b2 = off; off += kWsC * 4;
  l.bo = off; l.lg = off + kWsC * 4; l.lb = off + 2 * kWsC * 4;
  if (tail) off += 3 * kWsC * 4;
  l.wo = off;
  if (tail) off += kWsC * kWsC * 2;
  l.ctr = off; off += 16;
  l.bytes = off;
  return l;
}

template <bool TAIL>
__global__ __launch_bounds__(kWsThreads) void mlp_ws_kernel(MlpArgs A, int blk_per_wg) {
  constexpr int C = kWsC, KS = 2, OT = 4, SH = 1, MSK = 7;
  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int lq = lane & 15, lg = lane >> 4;
  const int T = A.T, Hd = A.Hd, nch = Hd / 32;
  const WsLayout L = ws_layout(nch, TAIL);
  float* b2s = (float*)(lds + L.b2);
  int* ctr = (int*)(lds + L.ctr);
  const uint32_t tbytes = (uint32_t)T * C * 2;
  const auto Xr = mlp_rsrc(A.x, tbytes);
  const auto Rr = mlp_rsrc(A.r, tbytes);
  const auto Or = mlp_rsrc(A.out, tbytes);
  const auto W1r = mlp_rsrc(A.w1, (uint32_t)Hd * C * 2);
  const auto W2r = mlp_rsrc(A.w2, (uint32_t)C * Hd * 2);

  // ---- stage every chunk (layouts as mlp_kernel's buffers) ----
  for (int e = tid; e < nch * 4 * C; e += kWsThreads) {
    const int j = e / (4 * C), k = e - j * 4 * C;
    uint16_t* W1s = (uint16_t*)(lds + j * kWsChunk);
    const int r = k / (C / 8), c = k % (C / 8);
    const int ca = TAIL ? 32 * (c >> 2) + 4 * (c & 3) : 8 * c;
    const int cb = TAIL ? ca + 16 : ca + 4;
    const uint32_t row = (uint32_t)(j * 32 + r) * C;
    const uint2 a = mload8(W1r, (row + ca) * 2), b = mload8(W1r, (row + cb) * 2);
    *(uint4*)(W1s + r * C + ((c ^ ((r >> SH) & MSK)) << 3)) = make_uint4(a.x, a.y, b.x, b.y);
  }
  for (int e = tid; e < nch * 4 * C; e += kWsThreads) {
    const int j = e / (4 * C), k = e - j * 4 * C;
    uint16_t* W2s = (uint16_t*)(lds + j * kWsChunk) + 32 * C;
    const int o = k >> 2, g = k & 3;
    const uint32_t base = (uint32_t)(o * Hd + j * 32 + 4 * g) * 2;
    const uint2 a = mload8(W2r, base), b = mload8(W2r, base + 32);
    *(uint4*)(W2s + o * 32 + ((g ^ ((o >> 2) & 3)) << 3)) = make_uint4(a.x, a.y, b.x, b.y);
  }
  for (int e = tid; e < nch * 32; e += kWsThreads) {
    float* b1s = (float*)(lds + (e >> 5) * kWsChunk + (32 * C + C * 32) * 2);
    b1s[e & 31] = A.b1 ? A.b1[e] : 0.f;
  }
  for (int c = tid; c < C; c += kWsThreads) b2s[c] = A.b2 ? A.b2[c] : 0.f;
  if constexpr (TAIL) {
    float* bos = (float*)(lds + L.bo);
    float* lgs = (float*)(lds + L.lg);
    float* lbs = (float*)(lds + L.lb);
    uint16_t* Wos = (uint16_t*)(lds + L.wo);
    const auto Wor = mlp_rsrc(A.wo, (uint32_t)C * C * 2);
    for (int e = tid; e < C * C / 8; e += kWsThreads) {
      const int r = e / (C / 8), c = e % (C / 8);
      *(uint4*)(Wos + r * C + ((c ^ ((r >> SH) & MSK)) << 3)) = mload16(Wor, (uint32_t)e * 16);
    }
    for (int c = tid; c < C; c += kWsThreads) {
      bos[c] = A.bo ? A.bo[c] : 0.f;
      lgs[c] = A.lng[c];
      lbs[c] = A.lnb[c];
    }
  }
  if (tid == 0) *ctr = 0;
  __syncthreads();

  // ---- the workgroup's blocks, claimed one at a time by its wavefronts ----
  const int nblk = (T + 15) >> 4;
  const int b0 = blockIdx.x * blk_per_wg;
  const int b1 = min(nblk, b0 + blk_per_wg);
  auto claim = [&]() -> int {
    int v = 0;
    if (lane == 0) v = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return b0 + __builtin_amdgcn_readfirstlane(v);
  };
  // inputs of block bk: the operands of x (TAIL: y) in natural channel
  // order, and the residual (TAIL: x1) in the MFMA layout
  auto xoff = [&](int bk, int s) -> uint32_t {
    const int t = bk * 16 + lq;
    return (bk < b1 && t < T) ? (uint32_t)(t * C + 32 * s + 8 * lg) * 2 : kMlpOob;
  };
  auto moff = [&](int bk, int o) -> uint32_t {
    const int t = bk * 16 + lq;
    return (bk < b1 && t < T) ? (uint32_t)(t * C + 16 * o + 4 * lg) * 2 : kMlpOob;
  };
  int bk = claim();
  uint4 xin[KS];
  uint2 rin[OT];
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2) xin[s2] = mload16(Xr, xoff(bk, s2));
#pragma unroll
  for (int o = 0; o < OT; ++o) rin[o] = mload8(Rr, moff(bk, o));
  while (bk < b1) {
    bf16x8 xo[KS];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) xo[s2] = __builtin_bit_cast(bf16x8, xin[s2]);
    uint2 res[OT];
#pragma unroll
    for (int o = 0; o < OT; ++o) res[o] = rin[o];
    const int cur = bk;
    // the next block's inputs, in flight while this one is computed
    bk = claim();
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) xin[s2] = mload16(Xr, xoff(bk, s2));
#pragma unroll
    for (int o = 0; o < OT; ++o) rin[o] = mload8(Rr, moff(bk, o));

    if constexpr (TAIL) {
      // ---- x2 = x1 + y W_out^T + b_out, rounded; n2 = LN2(x2), rounded ----
      const float* bos = (const float*)(lds + L.bo);
      const float* lgs = (const float*)(lds + L.lg);
      const float* lbs = (const float*)(lds + L.lb);
      const uint16_t* Wos = (const uint16_t*)(lds + L.wo);
      float v[OT][4];
#pragma unroll
      for (int o = 0; o < OT; ++o) {
        const float4 bo4 = *(const float4*)(bos + 16 * o + 4 * lg);
        f32x4 a = {bo4.x, bo4.y, bo4.z, bo4.w};
        const int row = 16 * o + lq;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
          const int c = 4 * s2 + lg;
          const bf16x8 w = *(const bf16x8*)(Wos + row * C + ((c ^ ((row >> SH) & MSK)) << 3));
          a = mfma16(w, xo[s2], a);
        }
        const uint32_t p0 = pack_bf16x2(a[0] + bf16_lo(res[o].x), a[1] + bf16_hi(res[o].x));
        const uint32_t p1 = pack_bf16x2(a[2] + bf16_lo(res[o].y), a[3] + bf16_hi(res[o].y));
        res[o] = make_uint2(p0, p1);
        v[o][0] = bf16_lo(p0); v[o][1] = bf16_hi(p0);
        v[o][2] = bf16_lo(p1); v[o][3] = bf16_hi(p1);
        if (A.x2) {
          const u32x2 st = {p0, p1};
          __builtin_amdgcn_raw_buffer_store_b64(st, mlp_rsrc(A.x2, tbytes), moff(cur, o), 0, 0);
        }
      }
      float sm = 0.f;
#pragma unroll
      for (int o = 0; o < OT; ++o) sm += (v[o][0] + v[o][1]) + (v[o][2] + v[o][3]);
      sm += xor16(sm);
      sm += xor32(sm);
      const float mean = sm / (float)C;
      float sq = 0.f;
#pragma unroll
      for (int o = 0; o < OT; ++o)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float d = v[o][e] - mean;
          sq = fmaf(d, d, sq);
        }
      sq += xor16(sq);
      sq += xor32(sq);
      const float rstd = 1.0f / sqrtf(sq / (float)C + A.eps);
      uint32_t np[OT][2];
#pragma unroll
      for (int o = 0; o < OT; ++o) {
        const float4 g4 = *(const float4*)(lgs + 16 * o + 4 * lg);
        const float4 b4 = *(const float4*)(lbs + 16 * o + 4 * lg);
        np[o][0] = pack_bf16x2((v[o][0] - mean) * rstd * g4.x + b4.x,
                               (v[o][1] - mean) * rstd * g4.y + b4.y);
        np[o][1] = pack_bf16x2((v[o][2] - mean) * rstd * g4.z + b4.z,
                               (v[o][3] - mean) * rstd * g4.w + b4.w);
        if (A.n2) {
          const u32x2 st = {np[o][0], np[o][1]};
          __builtin_amdgcn_raw_buffer_store_b64(st, mlp_rsrc(A.n2, tbytes), moff(cur, o), 0, 0);
        }
      }
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        xo[s2] = __builtin_bit_cast(
            bf16x8, make_uint4(np[2 * s2][0], np[2 * s2][1], np[2 * s2 + 1][0], np[2 * s2 + 1][1]));
    }

    // ---- the MLP over every chunk of the hidden layer ----
    f32x4 acc[OT];
#pragma unroll
    for (int o = 0; o < OT; ++o) acc[o] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < nch; ++j) {
      const unsigned char* bp = lds + j * kWsChunk;
      const uint16_t* W1s = (const uint16_t*)bp;
      const uint16_t* W2s = W1s + 32 * C;
      const float* b1s = (const float*)(bp + (32 * C + C * 32) * 2);
      f32x4 h[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float4 bt = *(const float4*)(b1s + 16 * t + 4 * lg);
        h[t] = f32x4{bt.x, bt.y, bt.z, bt.w};
        const int row = 16 * t + lq;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
          const int c = 4 * s2 + lg;
          const bf16x8 a = *(const bf16x8*)(W1s + row * C + ((c ^ ((row >> SH) & MSK)) << 3));
          h[t] = mfma16(a, xo[s2], h[t]);
        }
      }
      const uint32_t u0 = pack_bf16x2(gelu_as(h[0][0]), gelu_as(h[0][1]));
      const uint32_t u1 = pack_bf16x2(gelu_as(h[0][2]), gelu_as(h[0][3]));
      const uint32_t u2 = pack_bf16x2(gelu_as(h[1][0]), gelu_as(h[1][1]));
      const uint32_t u3 = pack_bf16x2(gelu_as(h[1][2]), gelu_as(h[1][3]));
      const bf16x8 hop = __builtin_bit_cast(bf16x8, make_uint4(u0, u1, u2, u3));
#pragma unroll
      for (int o = 0; o < OT; ++o) {
        const int row = 16 * o + lq;
        const bf16x8 a = *(const bf16x8*)(W2s + row * 32 + ((lg ^ ((row >> 2) & 3)) << 3));
        acc[o] = mfma16(a, hop, acc[o]);
      }
    }

    // ---- epilogue (as mlp_kernel's) ----
    const bool odd = lg & 1;
    const int t = cur * 16 + lq;
#pragma unroll
    for (int m = 0; m < OT / 2; ++m) {
      float f[2][4];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int o = 2 * m + q;
        const float4 b4 = *(const float4*)(b2s + 16 * o + 4 * lg);
        f[q][0] = acc[o][0] + b4.x + bf16_lo(res[o].x);
        f[q][1] = acc[o][1] + b4.y + bf16_hi(res[o].x);
        f[q][2] = acc[o][2] + b4.z + bf16_lo(res[o].y);
        f[q][3] = acc[o][3] + b4.w + bf16_hi(res[o].y);
      }
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(f[0][e]),
                                                         __float_as_uint(f[1][e]), false, false);
        if (odd) {
          v[e] = __uint_as_float(sw[0]);
          v[4 + e] = f[1][e];
        } else {
          v[e] = f[0][e];
          v[4 + e] = __uint_as_float(sw[1]);
        }
      }
      const int ch = 32 * m + (odd ? 16 + 4 * (lg - 1) : 4 * lg);
      const uint32_t off = t < T ? (uint32_t)(t * C + ch) * 2 : kMlpOob;
      const u32x4 x = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                       pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
      __builtin_amdgcn_raw_buffer_store_b128(x, Or, off, 0, 0);
    }
  }
}

template <bool TAIL>
hipError_t mlp_ws_launch(const MlpArgs& a, hipStream_t st) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const WsLayout l = ws_layout(a.Hd / 32, TAIL);
  const void* fn = reinterpret_cast<const void*>(&mlp_ws_kernel<TAIL>);
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, l.bytes);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mlp_ws_kernel<TAIL>, kWsThreads, l.bytes);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorNotSupported;
  const long long nblk = ((long long)a.T + 15) / 16;
  long long groups = (long long)cus * per_cu;
  if (groups > nblk) groups = nblk;
  const int per = (int)((nblk + groups - 1) / groups);
  groups = (nblk + per - 1) / per;
  hipLaunchKernelGGL((mlp_ws_kernel<TAIL>), dim3((unsigned)groups), dim3(kWsThreads), l.bytes, st,
                     a, per);
  return hipGetLastError();
}

bool mlp_shape_ok(long long T, int C, int Hd) {
  if (T <= 0 || Hd <= 0 || Hd % 32) return false;
  if (C != 64 && C != 128 && C != 256) return false;
  // buffer offsets are 32-bit
  return T * C * 2 < (long long)kMlpOob && (long long)Hd * C * 2 < (long long)kMlpOob;
}

}  // namespace

hipError_t launch_mlp(const void* x, long long T, int C, int Hd, const void* w1, const float* b1,
                      const void* w2, const float* b2, const void* resid, void* out,
                      hipStream_t st) {
  if (!mlp_shape_ok(T, C, Hd)) return hipErrorNotSupported;
  MlpArgs a = {};
  a.x = (const uint16_t*)x; a.w1 = (const uint16_t*)w1; a.b1 = b1;
  a.w2 = (const uint16_t*)w2; a.b2 = b2; a.r = (const uint16_t*)resid; a.out = (uint16_t*)out;
  a.T = (int)T; a.Hd = Hd;
  if (C == 64 && Hd <= 256) return mlp_ws_launch<false>(a, st);
  if (C == 64) return mlp_launch<Mg<64, 32>, false>(a, st);
  if (C == 128) return mlp_launch<Mg<128, 16>, false>(a, st);
  return mlp_launch<Mg<256, 16>, false>(a, st);
}

hipError_t launch_block_tail(const void* y, const void* x1, long long T, int C, int Hd,
                             const void* w_out, const float* b_out, const float* ln_g,
                             const float* ln_b, float eps, const void* w1, const float* b1,
                             const void* w2, const float* b2, void* x2, void* n2, void* out,
                             hipStream_t st) {
  // W_out stays in LDS beside the chunk buffers: C up to 128
  if (!mlp_shape_ok(T, C, Hd) || C > 128) return hipErrorNotSupported;
  MlpArgs a = {};
  a.x = (const uint16_t*)y; a.w1 = (const uint16_t*)w1; a.b1 = b1;
  a.w2 = (const uint16_t*)w2; a.b2 = b2; a.r = (const uint16_t*)x1; a.out = (uint16_t*)out;
  a.wo = (const uint16_t*)w_out; a.bo = b_out; a.lng = ln_g; a.lnb = ln_b; a.eps = eps;
  a.x2 = (uint16_t*)x2; a.n2 = (uint16_t*)n2;
  a.T = (int)T; a.Hd = Hd;
  if (C == 64 && Hd <= 256) return mlp_ws_launch<true>(a, st);
  if (C == 64) return mlp_launch<Mg<64, BRA_TAIL_TW64>, true>(a, st);
  return mlp_launch<Mg<128, 16>, true>(a, st);
}

}  // namespace bra
