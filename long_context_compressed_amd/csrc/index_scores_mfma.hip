// Matrix-core (MFMA) lightning-indexer scores on gfx950 for d_I = 128, H_I = 64:
//   I[t, j] = sum_h w[t,h] relu(qI[t,h] . kI[row0 + j]),  j < n_vis(p)
// ("DeepSeek-V4 Attention Training Systems", section 3 indexer logits; section 9: the
// indexer query is FP8-eligible).
//
// One wave per query token, 8 consecutive tokens per workgroup.  The token's 64 x 128
// indexer query is resident in registers as the MFMA A operand; each step multiplies it
// with 64 visible compressed keys (B operand), so the Z = qI kI^T tile [64 heads x 64 keys]
// lives in 16 accumulator tiles.  When the 8 tokens lie in one sample (they then see the
// same keys, up to one block), every 64-key block is gathered once into LDS for the whole
// workgroup (direct global->LDS loads, a block ahead) and all 8 waves read their B operands
// from there: the key bytes through the CU's load path drop 8-fold, which otherwise bound
// the kernel at about the MFMA rate.  Groups that straddle a sample boundary load the keys
// per wave (16-byte row loads).  ReLU, the per-(token, head) weight and the head sum are
// done in registers: 16 heads inside each lane, then the 4 lane groups via cross-lane adds,
// in a fixed order (deterministic; both paths sum alike).
//   bf16: v_mfma_f32_16x16x32_bf16, 4 k-steps per tile.
//   fp8 (OCP e4m3 codes): v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales, one
//   instruction per tile; the per-row fp32 scales of qI and kI multiply the result.
// The fused variant keeps each token's scores in a wave-private LDS row and runs the
// wave-level radix top-k on it, so the score matrix need not round-trip through HBM
// (section 8.2 lists fusing scores with top-k as open work).
#include "attn_common.h"
#include "csa_launch.h"
#include "topk_wave.h"

// M0 is named as clobbered by the LDS-DMA asm below; the compiler keeps no value in it here.
#pragma clang diagnostic ignored "-Winline-asm"

namespace csa {

using attn::bf16x8;
using attn::f32x4;
using attn::ld16;
using attn::swz;
using attn::token_info_wave;
typedef int i32x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int kHI = 64;
constexpr int kDI = 128;
constexpr int kSW = 8;    // tokens (waves) per workgroup
constexpr int kKB = 64;   // keys per block

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Four 256-byte key rows per instruction (global_load_lds_dwordx4): lane l's 16 bytes land
// at LDS byte offset lds + 16 l.  Issued through asm so that the compiler does not order LDS
// reads of the other buffer behind it; completion is awaited with wait_vmem().
__device__ __forceinline__ void dma_rows16(const void* src, const void* lds) {
  const uint32_t d = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(d), "v"(src) : "memory", "m0");
}

struct ScArgs {
  const void* qI;
  const float* qI_scale;
  const float* w;
  const void* kI;
  const float* kI_scale;
  const int32_t* cu;
  const int32_t* cu_cmp;
  float* scores;
  int64_t ld;
  int B, T, r, n_cap;
  int t_lo;   // first token of the stand-alone score kernel (its row t - t_lo of scores)
};

// Scores of one token's visible keys j < nv, 64 at a time: emit(j0, s) is called once per
// block with lane l holding the score of j = j0 + l (keys past nv hold unspecified values).
// The product for keys j0 + 16 nt + c16 finishes with the sum over the four lane groups in
// every group alike, so the lane of group g keeps its value from tile nt = g.  The wave
// takes blocks b0, b0 + bstride, ... (several waves may share one token's blocks).
template <bool FP8, class Emit>
__device__ __forceinline__ void score_blocks(const ScArgs& a, int t, int row0, int nv,
                                             Emit&& emit, int b0 = 0, int bstride = 1) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;

  // per-lane weights of the output rows h = 16mt + 4g + i (and fp8 query scales)
  float wv[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 16 * mt + 4 * g + i;
      float x = a.w[(int64_t)t * kHI + h];
      if (FP8) x *= a.qI_scale[(int64_t)t * kHI + h];
      wv[mt][i] = x;
    }

  if constexpr (!FP8) {
    const uint16_t* q = (const uint16_t*)a.qI + (int64_t)t * kHI * kDI;
    const uint16_t* k = (const uint16_t*)a.kI;
    bf16x8 qa[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qa[mt][ks] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(q + (16 * mt + c16) * kDI + 32 * ks + 8 * g));
    for (int j0 = kKB * b0; j0 < nv; j0 += kKB * bstride) {
      bf16x8 kb[4][4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int j = j0 + 16 * nt + c16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          uint4 v = make_uint4(0, 0, 0, 0);
          if (j < nv)
            v = *reinterpret_cast<const uint4*>(k + (int64_t)(row0 + j) * kDI + 32 * ks + 8 * g);
          kb[nt][ks] = __builtin_bit_cast(bf16x8, v);
        }
      }
      float mine = 0.f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float s = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][ks], kb[nt][ks], z, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) s = fmaf(wv[mt][i], fmaxf(z[i], 0.f), s);
        }
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        if (nt == g) mine = s;
      }
      emit(j0, mine + 0.0f);
    }
  } else {
    const uint8_t* q = (const uint8_t*)a.qI + (int64_t)t * kHI * kDI;
    const uint8_t* k = (const uint8_t*)a.kI;
    i32x8 qa[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint4* p = reinterpret_cast<const uint4*>(q + (16 * mt + c16) * kDI + 32 * g);
      const uint4 lo = p[0], hi = p[1];
      qa[mt] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    for (int j0 = kKB * b0; j0 < nv; j0 += kKB * bstride) {
      i32x8 kb[4];
      float ks_[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int j = j0 + 16 * nt + c16;
        uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
        float sc = 0.f;
        if (j < nv) {
          const uint4* p = reinterpret_cast<const uint4*>(k + (int64_t)(row0 + j) * kDI + 32 * g);
          lo = p[0];
          hi = p[1];
          sc = a.kI_scale[row0 + j];
        }
        kb[nt] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        ks_[nt] = sc;
      }
      float mine = 0.f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float s = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
          // unit block scales (E8M0 127 = 2^0), A and B in fp8 e4m3 (format 0)
          z = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[mt], kb[nt], z, 0, 0, 0, 127, 0,
                                                               127);
#pragma unroll
          for (int i = 0; i < 4; ++i) s = fmaf(wv[mt][i], fmaxf(z[i] * ks_[nt], 0.f), s);
        }
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        if (nt == g) mine = s;
      }
      emit(j0, mine + 0.0f);
    }
  }
}

// Whether the workgroup's kSW tokens t0 .. t0 + kSW - 1 are all real and in one sample
// (then they share key blocks): gives that sample's first compressed row and the visible
// count of its last token, the longest row of the group.  Wave-uniform, and the same in
// every wave of the workgroup.
__device__ __forceinline__ bool group_shares(const ScArgs& a, int t0, int& row0, int& nv_max) {
  const int tl = t0 + kSW - 1;
  if (tl >= a.T) return false;
  TokenInfo f, l;
  if (!token_info_wave(a.cu, a.B, t0, f, a.cu_cmp)) return false;
  if (!token_info_wave(a.cu, a.B, tl, l)) return false;
  if (f.b != l.b) return false;
  row0 = f.c0;
  nv_max = min((l.p + 1) / a.r, a.n_cap);
  return true;
}

// LDS of the shared key blocks: two buffers of 64 rows (256-byte bf16 rows, or 128-byte
// fp8 code rows and the rows' 64 fp32 scales).
template <bool FP8>
struct KeyTiles {
  uint8_t rows[2][kKB * kDI * 2];
};
template <>
struct KeyTiles<true> {
  uint8_t rows[2][kKB * kDI];
  float scale[2][kKB];
};

// 16-byte chunk swizzle of the fp8 128-byte rows: physical chunk = logical ^ swz8(row).  The
// sixteen rows of one MFMA column tile read at one logical chunk then fall in sixteen
// distinct 16-byte bank groups (row parity picks the half of the 64 banks).
__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }

// 64 fp32 key scales of a block (global_load_lds_dword): lane l's 4 bytes land at lds + 4 l.
__device__ __forceinline__ void dma_dword(const void* src, const void* lds) {
  const uint32_t d = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(d), "v"(src) : "memory", "m0");
}

// Scores of this wave's token (nv keys) with the workgroup's key blocks staged in LDS: every
// block of the group's longest row (nv_max keys) is gathered once, a block ahead, into
// swizzled rows, and read by every wave as the B operand (fp8: with the keys' scales).
// Every wave runs every block and its barrier; a wave with want = false, or whose row has
// ended, only helps with the gathers.  emit as in score_blocks, and the products, weights
// and head sums are formed in the same order as there.
template <bool FP8, class Emit>
__device__ __forceinline__ void score_blocks_lds(const ScArgs& a, int t, int row0, int nv,
                                                 bool want, int nv_max, KeyTiles<FP8>& kt,
                                                 Emit&& emit) {
  constexpr int kRowB = FP8 ? kDI : 2 * kDI;   // bytes per key row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  float wv[4][4];
  bf16x8 qa[4][4];   // bf16: [mt][ks]
  i32x8 q8[4];       // fp8: [mt]
  if (want) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 16 * mt + 4 * g + i;
        float x = a.w[(int64_t)t * kHI + h];
        if (FP8) x *= a.qI_scale[(int64_t)t * kHI + h];
        wv[mt][i] = x;
      }
    if constexpr (FP8) {
      const uint8_t* q = (const uint8_t*)a.qI + (int64_t)t * kHI * kDI;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const uint4* p = reinterpret_cast<const uint4*>(q + (16 * mt + c16) * kDI + 32 * g);
        const uint4 lo = p[0], hi = p[1];
        q8[mt] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    } else {
      const uint16_t* q = (const uint16_t*)a.qI + (int64_t)t * kHI * kDI;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qa[mt][ks] = ld16(q + (16 * mt + c16) * kDI + 32 * ks + 8 * g);
    }
  }
  const uint8_t* kg = (const uint8_t*)a.kI;
  const int nb = (nv_max + kKB - 1) / kKB;
  // bf16: wave w gathers rows 8w .. 8w+7, four per instruction (lane l fills physical chunk
  // l % 16 of row 4i + l / 16); fp8: eight rows in one instruction (chunk l % 8 of row
  // l / 8) and wave 0 also the 64 scales.  Rows past the group's longest row repeat its
  // last key (finite, never emitted).
  auto issue = [&](int b, int buf) {
    if constexpr (FP8) {
      const int r = 8 * wave + (lane >> 3);
      const int j = min(kKB * b + r, nv_max - 1);
      dma_rows16(kg + (int64_t)(row0 + j) * kDI + 16 * ((lane & 7) ^ swz8(r)),
                 &kt.rows[buf][8 * wave * kRowB]);
      if (wave == 0)
        dma_dword(a.kI_scale + row0 + min(kKB * b + lane, nv_max - 1), &kt.scale[buf][0]);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 8 * wave + 4 * i + (lane >> 4);
        const int j = min(kKB * b + r, nv_max - 1);
        dma_rows16(kg + (int64_t)(row0 + j) * kRowB + 16 * ((lane & 15) ^ swz(r)),
                   &kt.rows[buf][(8 * wave + 4 * i) * kRowB]);
      }
    }
  };
  if (nb > 0) issue(0, 0);
  for (int b = 0; b < nb; ++b) {
    const int buf = b & 1;
    wait_vmem();       // this wave's rows of block b
    __syncthreads();   // every wave's rows of block b; block b - 1's buffer is free
    if (b + 1 < nb) issue(b + 1, buf ^ 1);
    if (!want || kKB * b >= nv) continue;
    float mine = 0.f;
    if constexpr (FP8) {
      // B operand: key 16 nt + c16 (swz8 depends on c16 only), logical chunks 2g, 2g + 1
      const uint8_t* kr = &kt.rows[buf][c16 * kRowB];
      const int s8 = swz8(c16);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const uint4 lo = *reinterpret_cast<const uint4*>(kr + 16 * nt * kRowB + 16 * ((2 * g) ^ s8));
        const uint4 hi = *reinterpret_cast<const uint4*>(kr + 16 * nt * kRowB + 16 * ((2 * g + 1) ^ s8));
        const i32x8 kb = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                               (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        const float ksc = kt.scale[buf][16 * nt + c16];
        float s = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
          // unit block scales (E8M0 127 = 2^0), A and B in fp8 e4m3 (format 0)
          z = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q8[mt], kb, z, 0, 0, 0, 127, 0, 127);
#pragma unroll
          for (int i = 0; i < 4; ++i) s = fmaf(wv[mt][i], fmaxf(z[i] * ksc, 0.f), s);
        }
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        if (nt == g) mine = s;
      }
    } else {
      // B operand: key 16 nt + c16 (swz depends on the row's low 4 bits), logical chunk 4 ks + g
      const uint16_t* kr = reinterpret_cast<const uint16_t*>(&kt.rows[buf][c16 * kRowB]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        bf16x8 kb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kb[ks] = ld16(kr + 16 * nt * kDI + 8 * ((4 * ks + g) ^ swz(c16)));
        float s = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][ks], kb[ks], z, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) s = fmaf(wv[mt][i], fmaxf(z[i], 0.f), s);
        }
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        if (nt == g) mine = s;
      }
    }
    emit(kKB * b, mine + 0.0f);
  }
}

// Tokens t_lo .. T - 1 (T: the end of the range), score row t - t_lo.
template <bool FP8>
__global__ __launch_bounds__(kSW * 64) void k_index_scores_mfma(ScArgs a) {
  __shared__ __attribute__((aligned(16))) KeyTiles<FP8> kt;
  const int lane = threadIdx.x & 63;
  const int t0 = a.t_lo + blockIdx.x * kSW, t = t0 + (threadIdx.x >> 6);
  int row0 = 0, nv_max = 0;
  if (group_shares(a, t0, row0, nv_max)) {
    TokenInfo ti;
    token_info_wave(a.cu, a.B, t, ti);   // inside the group's sample
    const int nv = min((ti.p + 1) / a.r, a.n_cap);
    float* out = a.scores + (int64_t)(t - a.t_lo) * a.ld;
    score_blocks_lds<FP8>(a, t, row0, nv, nv > 0, nv_max, kt, [&](int j0, float s) {
      if (j0 + lane < nv) out[j0 + lane] = s;
    });
    return;
  }
  if (t >= a.T) return;
  TokenInfo ti;
  if (!token_info_wave(a.cu, a.B, t, ti, a.cu_cmp)) return;
  const int nv = min((ti.p + 1) / a.r, a.n_cap);
  if (nv <= 0) return;
  float* out = a.scores + (int64_t)(t - a.t_lo) * a.ld;
  score_blocks<FP8>(a, t, ti.c0, nv, [&](int j0, float s) {
    if (j0 + lane < nv) out[j0 + lane] = s;
  });
}

// Fused scores + top-k for rows of up to 64 * KPL visible keys, one wave per token: the
// scores go to a wave-private LDS row (plus HBM when mode 2 asks for all of them), then the
// wave's radix top-k selects from LDS and, in mode 1, stores the selected scores only.
// Rows with nv <= k select every visible key, and skip the scores unless they are wanted.
template <bool FP8, int KPL>
__global__ __launch_bounds__(kSW * 64) void k_index_topk(ScArgs a, int k, int k_cap, int mode,
                                                         int32_t* __restrict__ idx) {
  // each wave's score row, reused for its radix histograms once the keys are in registers
  constexpr int kSub = 8;
  constexpr int kRow = 64 * KPL > kSub * kHistStride ? 64 * KPL : kSub * kHistStride;
  __shared__ __attribute__((aligned(16))) float rows[kSW][kRow];
  __shared__ __attribute__((aligned(16))) KeyTiles<FP8> kt;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kSW, t = t0 + wave;
  int row0g = 0, nv_max = 0;
  const bool shared = group_shares(a, t0, row0g, nv_max);
  if (!shared && t >= a.T) return;
  int32_t* out = idx + (int64_t)t * k_cap;
  TokenInfo ti;
  const bool real = token_info_wave(a.cu, a.B, t, ti, a.cu_cmp);
  const int nv = real ? min((ti.p + 1) / a.r, a.n_cap) : 0;
  const int row0 = real ? ti.c0 : 0;
  float* srow = a.scores ? a.scores + (int64_t)t * a.ld : nullptr;
  float* lrow = rows[wave];
  if (shared) {
    // rows with nv <= k need their scores only when the loss reads them (mode != 0)
    score_blocks_lds<FP8>(a, t, row0, nv, nv > k || mode != 0, nv_max, kt, [&](int j0, float s) {
      if (j0 + lane < nv) {
        if (nv > k) {
          lrow[j0 + lane] = s;
          if (mode == 2) srow[j0 + lane] = s;
        } else {
          srow[j0 + lane] = s;
        }
      }
    });
  }
  if (nv <= k) {  // every visible row is selected (also covers padding rows: nv = 0)
    if (!shared && mode != 0 && nv > 0)
      score_blocks<FP8>(a, t, row0, nv, [&](int j0, float s) {
        if (j0 + lane < nv) srow[j0 + lane] = s;
      });
    for (int c = lane; c < k_cap; c += 64) out[c] = c < nv ? row0 + c : -1;
    return;
  }
  if (!shared)
    score_blocks<FP8>(a, t, row0, nv, [&](int j0, float s) {
      if (j0 + lane < nv) {
        lrow[j0 + lane] = s;
        if (mode == 2) srow[j0 + lane] = s;
      }
    });
  __builtin_amdgcn_wave_barrier();
  const int n_it = __builtin_amdgcn_readfirstlane((nv + 63) >> 6);
  float* sel = mode == 1 ? srow : nullptr;
  uint32_t* hist = reinterpret_cast<uint32_t*>(lrow);
  if (KPL >= 16 && n_it <= 16) topk_row_wave<16, kSub>(lrow, nv, n_it, k, row0, out, hist, sel);
  else if (KPL >= 32 && n_it <= 32) topk_row_wave<32, kSub>(lrow, nv, n_it, k, row0, out, hist, sel);
  else if (KPL >= 48 && n_it <= 48) topk_row_wave<48, kSub>(lrow, nv, n_it, k, row0, out, hist, sel);
  else topk_row_wave<(KPL > 48 ? 64 : KPL), kSub>(lrow, nv, n_it, k, row0, out, hist, sel);
  for (int c = k + lane; c < k_cap; c += 64) out[c] = -1;
}

// Fused scores + top-k for rows beyond 4096 visible keys (up to kTopkThreads * KPL), one
// workgroup of 8 waves per token: the waves score the token's 64-key blocks round robin
// (wave w takes blocks w, w + 8, ...; keys read per wave from L2, the same products as the
// other score kernels) into the workgroup's LDS row, and the workgroup radix top-k selects
// from it, so the row never leaves the chip.  Scores reach HBM only as mode asks (1: the
// selected ones, 2: every visible one).  Rows with nv <= k select every visible key and
// compute their scores only when the loss reads them.
template <bool FP8, int KPL>
__global__ __launch_bounds__(kTopkThreads) void k_index_topk_wg(ScArgs a, int k, int k_cap,
                                                                int mode,
                                                                int32_t* __restrict__ idx) {
  __shared__ __attribute__((aligned(16))) float lrow[kTopkThreads * KPL];
  __shared__ TopkWgLds<KPL> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NW = kTopkThreads / 64;
  const int t = blockIdx.x;
  int32_t* out = idx + (int64_t)t * k_cap;
  TokenInfo ti;
  const bool real = token_info_wave(a.cu, a.B, t, ti, a.cu_cmp);
  const int nv = real ? min((ti.p + 1) / a.r, a.n_cap) : 0;
  const int row0 = real ? ti.c0 : 0;
  float* srow = a.scores ? a.scores + (int64_t)t * a.ld : nullptr;
  if (nv <= k) {  // every visible row is selected (also covers padding rows: nv = 0)
    if (mode != 0 && nv > 0)
      score_blocks<FP8>(a, t, row0, nv, [&](int j0, float s) {
        if (j0 + lane < nv) srow[j0 + lane] = s;
      }, wave, NW);
    for (int c = tid; c < k_cap; c += kTopkThreads) out[c] = c < nv ? row0 + c : -1;
    return;
  }
  score_blocks<FP8>(a, t, row0, nv, [&](int j0, float s) {
    if (j0 + lane < nv) {
      lrow[j0 + lane] = s;
      if (mode == 2) srow[j0 + lane] = s;
    }
  }, wave, NW);
  __syncthreads();
  const int n_it = (nv + kTopkThreads - 1) / kTopkThreads;
  topk_row_wg<KPL>(lrow, nv, n_it, k, row0, out, sm, mode == 1 ? srow : nullptr);
  for (int c = k + tid; c < k_cap; c += kTopkThreads) out[c] = -1;
}

}  // namespace

hipError_t launch_index_scores_mfma(const Shape& sh, const void* qI, const float* qI_scale,
                                    const float* w, const void* kI, const float* kI_scale,
                                    float* scores, int64_t ld, hipStream_t s, bool* handled,
                                    int t_lo, int t_hi) {
  *handled = false;
  if (sh.HI != kHI || sh.dI != kDI || sh.idx_dtype == 0) return hipSuccess;
  *handled = true;
  if (t_hi < 0) t_hi = sh.T;
  if (t_hi <= t_lo) return hipSuccess;
  ScArgs a;
  a.qI = qI;
  a.qI_scale = qI_scale;
  a.w = w;
  a.kI = kI;
  a.kI_scale = kI_scale;
  a.cu = sh.cu;
  a.cu_cmp = sh.cu_cmp;
  a.scores = scores;
  a.ld = ld;
  a.B = sh.B;
  a.T = t_hi;
  a.r = sh.r;
  a.n_cap = sh.max_seqlen / sh.r;
  a.t_lo = t_lo;
  const unsigned grid = (unsigned)((t_hi - t_lo + kSW - 1) / kSW);
  if (sh.idx_dtype == 2)
    hipLaunchKernelGGL(k_index_scores_mfma<true>, dim3(grid), dim3(kSW * 64), 0, s, a);
  else
    hipLaunchKernelGGL(k_index_scores_mfma<false>, dim3(grid), dim3(kSW * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_index_topk(const Shape& sh, const void* qI, const float* qI_scale,
                             const float* w, const void* kI, const float* kI_scale,
                             int scores_mode, float* scores, int64_t ld, int32_t* idx,
                             hipStream_t s, bool* handled) {
  *handled = false;
  const int n_cap = sh.max_seqlen / sh.r;
  if (sh.HI != kHI || sh.dI != kDI || sh.idx_dtype == 0 || n_cap > kTopkThreads * 64)
    return hipSuccess;
  *handled = true;
  if (sh.T == 0) return hipSuccess;
  ScArgs a;
  a.qI = qI;
  a.qI_scale = qI_scale;
  a.w = w;
  a.kI = kI;
  a.kI_scale = kI_scale;
  a.cu = sh.cu;
  a.cu_cmp = sh.cu_cmp;
  a.scores = scores_mode != 0 ? scores : nullptr;
  a.ld = ld;
  a.B = sh.B;
  a.T = sh.T;
  a.r = sh.r;
  a.n_cap = n_cap;
  a.t_lo = 0;
  const bool fp8 = sh.idx_dtype == 2;
  if (n_cap > 64 * 64) {   // rows beyond a wave's 4096 keys: a workgroup per token
    const dim3 grid_w(sh.T), block_w(kTopkThreads);
#define CSA_LAUNCH_FUSED_WG(F, K)                                                              \
  hipLaunchKernelGGL((k_index_topk_wg<F, K>), grid_w, block_w, 0, s, a, sh.k, sh.k_cap,       \
                     scores_mode, idx)
    if (n_cap <= kTopkThreads * 16) {
      if (fp8) CSA_LAUNCH_FUSED_WG(true, 16); else CSA_LAUNCH_FUSED_WG(false, 16);
    } else if (n_cap <= kTopkThreads * 32) {
      if (fp8) CSA_LAUNCH_FUSED_WG(true, 32); else CSA_LAUNCH_FUSED_WG(false, 32);
    } else {
      if (fp8) CSA_LAUNCH_FUSED_WG(true, 64); else CSA_LAUNCH_FUSED_WG(false, 64);
    }
#undef CSA_LAUNCH_FUSED_WG
    return hipGetLastError();
  }
  const dim3 grid((sh.T + kSW - 1) / kSW), block(kSW * 64);
#define CSA_LAUNCH_FUSED(F, K)                                                                 \
  hipLaunchKernelGGL((k_index_topk<F, K>), grid, block, 0, s, a, sh.k, sh.k_cap, scores_mode, idx)
  if (n_cap <= 64 * 16) {
    if (fp8) CSA_LAUNCH_FUSED(true, 16); else CSA_LAUNCH_FUSED(false, 16);
  } else if (n_cap <= 64 * 32) {
    if (fp8) CSA_LAUNCH_FUSED(true, 32); else CSA_LAUNCH_FUSED(false, 32);
  } else {
    if (fp8) CSA_LAUNCH_FUSED(true, 64); else CSA_LAUNCH_FUSED(false, 64);
  }
#undef CSA_LAUNCH_FUSED
  return hipGetLastError();
}

}  // namespace csa
