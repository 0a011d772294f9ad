// Indexer KL loss with the dense (all visible compressed entries) teacher recomputed, for
// bf16 main operands (H = 64, D = 512) and a 64 x 128 indexer in bf16 or fp8, on gfx950.
//
// "DeepSeek-V4 Attention Training Systems", section 3: in the dense-loss warm-up the KL
// set C_t is the whole visible compressed history; the teacher is detached and the
// gradients reach the indexer query, head weights and indexer keys only.  Section 8.2:
// teacher scores are recomputed and the indexer backward runs eagerly, scaled by the
// caller's loss scale.  Teacher reading: P_t = mean over heads of the per-head softmax.
//
// The dense teacher costs 2 D H FLOP per (query, visible entry) and pass, against 1 KiB
// of key row: read per query, as the selected-set kernels do, it is bound by the row
// gathers.  Here the work is split three ways so each shared operand is read once per
// tile instead of once per (query, entry):
//   k_kld_teacher  one workgroup per 4 consecutive queries of one sample, two waves per
//                  query (32 heads each) with Q resident; each 64-row key block is loaded once
//                  into LDS (direct global->LDS loads, one row per S^T k-step, a block
//                  ahead) and feeds all 4 queries.  Pass 1: per-head online log-sum-exp
//                  of the teacher and the student log-sum-exp; pass 2: P (head mean), Q,
//                  KL_t and g = grad_scale (Q - P), written to the workspace.
//   k_kld_queries  the same 4-query groups, two waves per query (32 indexer heads each)
//                  with its qI resident; each 64-key block of kI is staged once into LDS for
//                  the 4 queries; z^T, E = g w 1[z > 0] (kept in registers as the A operand),
//                  dw and dqI = E kI.
//   k_kld_keys     one workgroup per (4 key blocks, query range), two waves per block (32
//                  indexer heads each); each query's qI tile is staged once into LDS for the 4
//                  blocks; z, E and dkI += E^T qI accumulate in registers over the range, one
//                  fp32 atomic add per key element and head half at the end.
// Queries are processed in chunks of kChunkRows (the workspace holds g for one chunk).
#include <math.h>

#include "attn_common.h"
#include "csa_launch.h"

// M0 is named as clobbered by the LDS-DMA asm below; the compiler keeps no value in it here.
#pragma clang diagnostic ignored "-Winline-asm"

namespace csa {

using namespace attn;

namespace {

constexpr int kHI = 64, kDI = 128;
constexpr int kKB = 64;            // key rows per block
constexpr int kChunkRows = 8192;   // queries per chunk
constexpr int kRange = 256;        // queries per key-gradient workgroup
constexpr int kIS = kDI + 8;       // bf16 row stride of the indexer tiles
constexpr int kI8S = kDI + 16;     // byte row stride of the fp8 code tiles
constexpr float kLazy = 8.f;
constexpr int kMaxBlocks = 512;    // key blocks of a row: n_cap <= 32768

typedef int i32x8 __attribute__((ext_vector_type(8)));

struct KldArgs {
  const uint16_t* q;
  const uint16_t* kv_cmp;
  const float* scores;      // student scores, row t - s_t0
  int64_t ld;
  int s_t0;
  const void* qI;
  const float* qI_scale;
  const uint16_t* qI16;   // bf16 indexer query rows from q16_t0 (the dequantized copy for fp8)
  int q16_t0;
  const float* w;
  const void* kI;
  const float* kI_scale;
  const uint16_t* kI16;   // fp8: bf16 copy of the indexer keys
  const int32_t* cu;
  const int32_t* cu_cmp;
  float* g;               // [kChunkRows, n_cap]: g of query t at row t - t_lo
  float* kl;
  float* dqI;
  float* dw;
  float* dkI;
  float gs, scale_log2;
  int B, T, r, n_cap, t_lo, t_hi, tc_blocks, fp8;
};

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One 16-byte-per-lane global -> LDS load: lane l's 16 bytes (scalar row base + per-lane
// offset) land at LDS byte address lds + 16 l.  Completion is awaited with wait_vmem().
__device__ __forceinline__ void dma_row16_s(uint64_t row, uint32_t lane_off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds), "v"(lane_off), "s"(row) : "memory", "m0");
}

// The queries of workgroup bid of a chunk: regular groups are 4 consecutive queries from a
// 4-aligned row t0, cut at the end of t0's sample; the first (unaligned) queries of sample
// b = bid - kChunkRows / 4 form one more group.  Every query of the chunk falls in exactly
// one group, and a group never spans two samples.
__device__ __forceinline__ bool query_group(const KldArgs& a, int bid, int& t_first, int& n,
                                            TokenInfo& ti) {
  int t0, lim;
  if (bid < kChunkRows / 4) {
    t0 = a.t_lo + 4 * bid;
    if (t0 >= a.t_hi || !token_info(a.cu, a.B, t0, ti)) return false;
    lim = min(t0 + 4, ti.start + ti.len);
  } else {
    const int b = bid - kChunkRows / 4;
    if (b >= a.B) return false;
    const int s = a.cu[b], e = a.cu[b + 1];
    if ((s & 3) == 0 || s == e || s < a.t_lo || s >= a.t_hi) return false;
    t0 = s;
    lim = min((s + 3) & ~3, e);
    if (!token_info(a.cu, a.B, t0, ti)) return false;
  }
  t_first = t0;
  n = min(lim, a.t_hi) - t0;
  return n > 0;
}

}  // namespace

// ---------------------------------------------------------------------------- teacher
// 8 waves: wave w serves query w / 2 of the group with heads 32 (w % 2) .. + 31, so two
// waves share each SIMD and one's softmax arithmetic overlaps the other's MFMAs.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_kld_teacher(KldArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[2][kKB][kD];
  __shared__ float Is[4][kKB];
  __shared__ float Ps[4][2][kKB];
  __shared__ float2 stu_s[4][kMaxBlocks];   // per query and key block: (max, sum of exp(I - max))

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int tw = wave >> 1, hh = wave & 1;
  if ((int)blockIdx.x < kChunkRows / 4 && tid < 4) {   // capacity padding rows: kl = 0
    const int u = a.t_lo + 4 * blockIdx.x + tid;
    if (u < a.t_hi && u >= a.cu[a.B]) a.kl[u] = 0.f;
  }
  int t_first, n_tok;
  TokenInfo ti;
  if (!query_group(a, blockIdx.x, t_first, n_tok, ti)) return;
  const bool active = tw < n_tok;
  const int t = t_first + (active ? tw : 0);
  const int row0 = __builtin_amdgcn_readfirstlane(a.cu_cmp[ti.b]);
  const int nv_w = active ? min((ti.p + tw + 1) / a.r, a.n_cap) : 0;
  const int nv_max = __builtin_amdgcn_readfirstlane(min((ti.p + n_tok) / a.r, a.n_cap));
  if (nv_max == 0) {
    if (active && hh == 0 && lane == 0) a.kl[t] = 0.f;
    return;
  }
  const int nblk = (nv_max + kKB - 1) / kKB;
  const float* srow = a.scores + (int64_t)(t - a.s_t0) * a.ld;
  float* grow = a.g + (int64_t)(t - a.t_lo) * a.n_cap;

  // Q rows as the A operand: qb[ht][ks] = Q[32 hh + 16 ht + c16][32 ks + 8 g .. +7]
  bf16x8 qb[2][16];
  {
    const uint16_t* qt = a.q + ((int64_t)t * kH + 32 * hh + c16) * kD + 8 * g;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qb[nt][ks] = ld16(qt + 16 * nt * kD + 32 * ks);
  }

  // key rows of a block: row 8 wave + j of block jb is visible row 64 jb + 8 wave + j
  // (row0 for slots past the last query's visible range: finite, masked below)
  const uint32_t lane16 = 16u * (uint32_t)lane;
  const uint32_t tile_lds = (uint32_t)(uintptr_t)&tile[0][0][0];
  auto gather = [&](int jb, int buf, int j) {
    const int r = 8 * wave + j;
    const int key = kKB * jb + r;
    const int row = __builtin_amdgcn_readfirstlane(row0 + (key < nv_max ? key : 0));
    const uint64_t src = (uint64_t)(uintptr_t)(a.kv_cmp + (int64_t)row * kD);
    const uint32_t lds = __builtin_amdgcn_readfirstlane(tile_lds + buf * (kKB * kD * 2) + r * (kD * 2));
    dma_row16_s(src, lane16 ^ (16u * swz(r)), lds);
  };
  int eq[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) eq[q] = 8 * ((4 * q + g) ^ swz(c16));

  // pass-1 state: per-head (m, l) of the lane's 8 heads 32 hh + 16 ht + 4 g + i over its
  // keys, and the student (m, l) over the whole row (the same in every lane)
  float m_run[8], l_run[8], lse2[8];
#pragma unroll
  for (int hx = 0; hx < 8; ++hx) { m_run[hx] = -INFINITY; l_run[hx] = 0.f; lse2[hx] = 0.f; }
  // the student normalizer, the KL terms and the teacher's total mass Z = sum_j P_j are
  // accumulated in fp64: the loss is A / Z - log Z with A = sum_j P_j (log P_j - log Q_j),
  // the KL of P / Z, so neither the fp32 rounding of the per-head normalizers (sum_j P_j =
  // 1 + O(1e-7)) nor that of a long fp32 sum biases a KL of near-uniform distributions
  float ms = -INFINITY, lseS = 0.f, lsum_f = 0.f, kl_acc = 0.f, z_acc = 0.f;

  for (int j = 0; j < 8; ++j) gather(0, 0, j);
  wait_vmem();
  __syncthreads();

  const int n_items = 2 * nblk;
  for (int it = 0; it < n_items; ++it) {
    const int buf = it & 1;
    const bool pass2 = it >= nblk;
    const int jb = pass2 ? it - nblk : it;
    const bool more = it + 1 < n_items;
    const int jb_next = it + 1 == nblk ? 0 : jb + 1;

    // scores of this block's keys (one per lane, coalesced), for the student
    float iv = -INFINITY;
    {
      const int j = kKB * jb + lane;
      if (j < nv_w) iv = srow[j];
    }

    // ---- S[head 32 hh + 16 ht + 4 g + i][key 16 kt + c16] over the block: Q rows are the
    // A operand (registers), key row segments the B operand (LDS)
    f32x4 acc[4][2];   // [kt][ht]
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) acc[kt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      const uint16_t* rb = &tile[buf][c16][0];
      auto seg = [&](int ks, int kt) { return ld16(rb + 16 * kt * kD + 128 * (ks >> 2) + eq[ks & 3]); };
      // (the other wave on the SIMD covers the LDS read latency: no software prefetch)
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        bf16x8 kb[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) kb[kt] = seg(ks, kt);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int ht = 0; ht < 2; ++ht) acc[kt][ht] = mfma16(qb[ht][ks], kb[kt], acc[kt][ht]);
        if (more && (ks & 1) == 0) gather(jb_next, buf ^ 1, ks >> 1);
      }
    }
    const int kbase = kKB * jb + c16;   // key of tile kt: kbase + 16 kt
    if (!pass2) {
      // ---- teacher: per lane, lazily rescaled online (max, sum) of its 8 heads over its keys
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int hx = 4 * ht + i;
          float bm = -INFINITY;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
            if (kbase + 16 * kt < nv_w) bm = fmaxf(bm, acc[kt][ht][i] * a.scale_log2);
          if (bm > m_run[hx] + kLazy) {
            l_run[hx] *= __builtin_amdgcn_exp2f(m_run[hx] - bm);
            m_run[hx] = bm;
          }
          if (m_run[hx] != -INFINITY) {
            float add = 0.f;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
              if (kbase + 16 * kt < nv_w)
                add += __builtin_amdgcn_exp2f(acc[kt][ht][i] * a.scale_log2 - m_run[hx]);
            l_run[hx] += add;
          }
        }
      // ---- student: online (max, sum) of the scores (natural log), lane = key
      {
        // each block's (max, sum) is recorded and the blocks are combined in fp64 once pass
        // 1 ends (an fp32 running sum over hundreds of blocks would drift)
        const float bm = wave_max(iv);
        const float bs = bm == -INFINITY ? 0.f : wave_sum(iv == -INFINITY ? 0.f : expf(iv - bm));
        if (hh == 0 && lane == 0) stu_s[tw][jb] = make_float2(bm, bs);
      }
      if (it == nblk - 1) {
        // merge the 16 lanes (keys) of each head; the student normalizer to every lane
#pragma unroll
        for (int hx = 0; hx < 8; ++hx) {
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) {
            const float mo = __shfl_xor(m_run[hx], o, 64), lo = __shfl_xor(l_run[hx], o, 64);
            const float mn = fmaxf(m_run[hx], mo);
            if (mn != -INFINITY) {
              l_run[hx] = l_run[hx] * __builtin_amdgcn_exp2f(m_run[hx] - mn) +
                          lo * __builtin_amdgcn_exp2f(mo - mn);
              m_run[hx] = mn;
            }
          }
          lse2[hx] = l_run[hx] > 0.f ? m_run[hx] + __log2f(l_run[hx]) : INFINITY;
        }
        __syncthreads();   // every query's block records
        {
          float m = -INFINITY;
          for (int b = lane; b < nblk; b += 64) m = fmaxf(m, stu_s[tw][b].x);
          ms = wave_max(m);
          double l = 0.0;
          if (ms != -INFINITY)
            for (int b = lane; b < nblk; b += 64) {
              const float2 v = stu_s[tw][b];
              if (v.x != -INFINITY) l += (double)(v.y * expf(v.x - ms));
            }
          l = wave_sum_f64(l);
          lsum_f = (float)l;
          lseS = l > 0.0 ? ms + logf(lsum_f) : INFINITY;
        }
      }
    } else {
      // ---- P = mean over heads of exp2(s - lse2): the lane's 8 heads in registers, the 4
      // lane groups by two exchanges, the two head halves through LDS
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        float p = 0.f;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            p += __builtin_amdgcn_exp2f(acc[kt][ht][i] * a.scale_log2 - lse2[4 * ht + i]);
        p += __shfl_xor(p, 16, 64);
        p += __shfl_xor(p, 32, 64);
        if (g == 0) Ps[tw][hh][16 * kt + c16] = p;
      }
      __syncthreads();
      // one key per lane (wave hh = 0 of each query): P, Q, the KL term and g
      if (hh == 0) {
        float gv = 0.f;
        if (kKB * jb + lane < nv_w) {
          const float P = (Ps[tw][0][lane] + Ps[tw][1][lane]) * (1.f / kH);
          const float logQ = iv - lseS;
          const float Q = expf(logQ);
          // log P - log Q = log(P * l_S) - (I - m_S): no cancellation of two logs of the
          // candidate count when both distributions are close to uniform
          if (P > 0.f) {
            kl_acc += P * (logf(P * lsum_f) - (iv - ms));
            z_acc += P;
          }
          gv = a.gs * (Q - P);
        }
        const int j = kKB * jb + lane;
        if (active && j < nv_w) grow[j] = gv;
      }
    }
    wait_vmem();
    __syncthreads();
  }
  if (active && hh == 0) {
    const double v = wave_sum_f64((double)kl_acc), z = wave_sum_f64((double)z_acc);
    if (lane == 0) a.kl[t] = z > 0.0 ? (float)(v / z - log1p(z - 1.0)) : 0.f;
  }
}

// ---------------------------------------------------------------------------- dkI
// Workgroup (x, y): 4 key blocks of 64 rows of one sample (regular groups start at
// 256-aligned rows and stop at the sample end; group tc_groups + b holds the first
// unaligned rows of sample b); 8 waves, wave w owning block w / 2 for indexer heads
// 32 (w % 2) .. + 31 (two waves per SIMD; each adds its head half of the block's dkI);
// queries y kRange .. of the chunk from the first one that sees the group's first key.  Each
// query's indexer query tile is staged once into LDS (double-buffered, fetched a query
// ahead) for the 4 blocks.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_kld_keys(KldArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t QIt[2][kHI][kIS];
  __shared__ __attribute__((aligned(16))) uint8_t QI8[2][kHI][kI8S];
  __shared__ __attribute__((aligned(16))) uint16_t KIt[4][kKB][kIS];   // bf16 indexer only
  __shared__ __attribute__((aligned(16))) uint8_t KI8[4][kKB][kI8S];   // fp8 codes only

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int kb = wave >> 1, hh = wave & 1;
  constexpr int kGroup = 4 * kKB;
  const int Tc = a.cu_cmp[a.B];
  int r_lo, r_hi, b;
  if ((int)blockIdx.x < a.tc_blocks) {
    r_lo = kGroup * blockIdx.x;
    if (r_lo >= Tc) return;
    b = upper_bound_i32(a.cu_cmp, a.B + 1, r_lo) - 1;
    r_hi = min(r_lo + kGroup, a.cu_cmp[b + 1]);
  } else {
    b = blockIdx.x - a.tc_blocks;
    if (b >= a.B) return;
    r_lo = a.cu_cmp[b];
    r_hi = min((r_lo + kGroup - 1) & ~(kGroup - 1), a.cu_cmp[b + 1]);
    if ((r_lo & (kGroup - 1)) == 0 || r_hi <= r_lo) return;
  }
  const int s_b = a.cu[b], e_b = a.cu[b + 1];
  const int jl0 = r_lo - a.cu_cmp[b];                 // first key, local to the sample
  const int t_min = s_b + a.r * (jl0 + 1) - 1;        // first query that sees it
  const int q_lo = max(max(t_min, a.t_lo + kRange * (int)blockIdx.y), s_b);
  const int q_hi = min(min(e_b, a.t_hi), a.t_lo + kRange * ((int)blockIdx.y + 1));
  if (q_lo >= q_hi) return;
  // this wave's block: keys jw .. jw + nk - 1 (local), rows r_lo + 64 kb ..
  const int jw = jl0 + kKB * kb;
  const int nk = max(0, min(kKB, r_hi - (r_lo + kKB * kb)));

  // the block's bf16 rows (or fp8 codes), rows past nk zero, loaded by its two waves (rows
  // 32 hh .. 32 hh + 31 each); every load of a lane is issued before its first store
  {
    constexpr int kPL = (kKB / 2) * (kDI / 8) / 64;   // 16-byte chunks per lane
    uint4 kv[kPL];
#pragma unroll
    for (int u = 0; u < kPL; ++u) {
      const int e = lane + 64 * u, row = 32 * hh + (e >> 4), ch = e & 15;
      const int64_t src = (int64_t)(r_lo + kKB * kb + row) * kDI;
      kv[u] = make_uint4(0, 0, 0, 0);
      if (row < nk) {
        if (!a.fp8) kv[u] = *reinterpret_cast<const uint4*>((const uint16_t*)a.kI + src + 8 * ch);
        else if (ch < 8) kv[u] = *reinterpret_cast<const uint4*>((const uint8_t*)a.kI + src + 16 * ch);
      }
    }
#pragma unroll
    for (int u = 0; u < kPL; ++u) {
      const int e = lane + 64 * u, row = 32 * hh + (e >> 4), ch = e & 15;
      if (!a.fp8) *reinterpret_cast<uint4*>(&KIt[kb][row][8 * ch]) = kv[u];
      else if (ch < 8) *reinterpret_cast<uint4*>(&KI8[kb][row][16 * ch]) = kv[u];
    }
  }

  // query tiles: 16 KiB of bf16 rows (2 chunks per thread) and 8 KiB of fp8 codes (1)
  uint4 pq[2], pq8;
  float pg[4], pw[2][4];   // the fetched query's g of the wave's keys 16 nt + c16, its w
  auto fetch = [&](int tq) {
    const int nvq = min((tq - s_b + 1) / a.r, a.n_cap);
    const float* grq = a.g + (int64_t)(tq - a.t_lo) * a.n_cap + jw;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int kj = 16 * nt + c16;
      pg[nt] = (kj < nk && jw + kj < nvq) ? grq[kj] : 0.f;
    }
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[m2][i] = a.w[(int64_t)tq * kHI + 32 * hh + 16 * m2 + 4 * g + i];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 512 * u, hr = e >> 4, ch = e & 15;
      pq[u] = *reinterpret_cast<const uint4*>(a.qI16 + ((int64_t)(tq - a.q16_t0) * kHI + hr) * kDI + 8 * ch);
    }
    if (a.fp8) {
      const int hr = tid >> 3, ch = tid & 7;
      pq8 = *reinterpret_cast<const uint4*>((const uint8_t*)a.qI + ((int64_t)tq * kHI + hr) * kDI + 16 * ch);
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 512 * u, hr = e >> 4, ch = e & 15;
      *reinterpret_cast<uint4*>(&QIt[buf][hr][8 * ch]) = pq[u];
    }
    if (a.fp8) {
      const int hr = tid >> 3, ch = tid & 7;
      *reinterpret_cast<uint4*>(&QI8[buf][hr][16 * ch]) = pq8;
    }
  };

  // dkI partial sums over this wave's heads: acc[nt][dt] = keys 16 nt + 4 g + i of the
  // wave's block, d 16 dt + c16
  f32x4 acc[4][8];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int jr = c16 >> 2, jc = 4 * (c16 & 3);
  const int ks = hh;   // k-step of the dkI product: head tiles 2 ks, 2 ks + 1

  fetch(q_lo);
  commit(0);
  for (int tq = q_lo; tq < q_hi; ++tq) {
    const int buf = (tq - q_lo) & 1;
    __syncthreads();
    float gvs[4], wv[2][4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) gvs[nt] = pg[nt];
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[m2][i] = pw[m2][i];
    if (tq + 1 < q_hi) fetch(tq + 1);
    const int nv_t = min((tq - s_b + 1) / a.r, a.n_cap);
    if (nk > 0 && nv_t > jw) {
      // z[head 16 mt + 4 g + i][key 16 nt + c16] for the wave's head tiles mt = 2 ks, 2 ks + 1
      // (the ReLU mask needs only its sign, so fp8 codes need no scales), then E = g w
      // 1[z > 0] as the bf16 A operand of the dkI product over those 32 heads; the qI rows
      // are read transposed in the same order
      bf16x8 qbt[8];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        qbt[dt] = join8(ld_tr(&QIt[buf][32 * ks + 4 * g + jr][16 * dt + jc]),
                        ld_tr(&QIt[buf][32 * ks + 16 + 4 * g + jr][16 * dt + jc]));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float gv = gvs[nt];
        uint32_t e4[4];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int mt = 2 * ks + h2;
          f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
          if (!a.fp8) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
              z = mfma16(ld16(&QIt[buf][16 * mt + c16][32 * kk + 8 * g]),
                         ld16(&KIt[kb][16 * nt + c16][32 * kk + 8 * g]), z);
          } else {
            const uint4* qp = reinterpret_cast<const uint4*>(&QI8[buf][16 * mt + c16][32 * g]);
            const uint4* kp = reinterpret_cast<const uint4*>(&KI8[kb][16 * nt + c16][32 * g]);
            const uint4 q0 = qp[0], q1 = qp[1], k0 = kp[0], k1 = kp[1];
            z = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                i32x8{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w},
                i32x8{(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w, (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w},
                z, 0, 0, 0, 127, 0, 127);
          }
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const float e0 = z[i] > 0.f ? gv * wv[h2][i] : 0.f;
            const float e1 = z[i + 1] > 0.f ? gv * wv[h2][i + 1] : 0.f;
            e4[2 * h2 + (i >> 1)] = pack_bf16x2(e0, e1);
          }
        }
        const bf16x8 ea = __builtin_bit_cast(bf16x8, make_uint4(e4[0], e4[1], e4[2], e4[3]));
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[nt][dt] = mfma16(ea, qbt[dt], acc[nt][dt]);
      }
    }
    if (tq + 1 < q_hi) commit(buf ^ 1);
  }
  // each wave adds its partial sums (rows past the block are skipped)
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kj = 16 * nt + 4 * g + i;
      if (kj < nk) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          atomicAdd(a.dkI + (int64_t)(r_lo + kKB * kb + kj) * kDI + 16 * dt + c16, acc[nt][dt][i]);
      }
    }
}

// ---------------------------------------------------------------------------- dqI, dw
// 8 waves: wave w serves query w / 2 of the group with indexer heads 32 (w % 2) .. + 31, so two
// waves share each SIMD and one's ReLU/E arithmetic overlaps the other's MFMAs.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_kld_queries(KldArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t KIt[2][kKB][kIS];
  __shared__ __attribute__((aligned(16))) uint8_t KI8[2][kKB][kI8S];
  __shared__ float ksc_s[2][kKB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int qw = wave >> 1, hh = wave & 1;
  if ((int)blockIdx.x < kChunkRows / 4) {   // capacity padding rows: dqI = 0, dw = 0
    const int u = a.t_lo + 4 * blockIdx.x + qw;
    if (u < a.t_hi && u >= a.cu[a.B]) {
      for (int e = lane; e < kHI * kDI / 2; e += 64)
        a.dqI[(int64_t)u * kHI * kDI + hh * (kHI * kDI / 2) + e] = 0.f;
      if (lane < kHI / 2) a.dw[(int64_t)u * kHI + 32 * hh + lane] = 0.f;
    }
  }
  int t_first, n_tok;
  TokenInfo ti;
  if (!query_group(a, blockIdx.x, t_first, n_tok, ti)) return;
  const bool active = qw < n_tok;
  const int t = t_first + (active ? qw : 0);
  const int row0 = a.cu_cmp[ti.b];
  const int nv_w = active ? min((ti.p + qw + 1) / a.r, a.n_cap) : 0;
  const int nv_max = min((ti.p + n_tok) / a.r, a.n_cap);
  const int nblk = (nv_max + kKB - 1) / kKB;
  const float* grow = a.g + (int64_t)(t - a.t_lo) * a.n_cap;

  // resident: qI^T as B operands (heads 32 hh + 16 nt + c16), head weights, fp8 row scales
  bf16x8 qb[2][4];
  i32x8 q8[2];
  float wv[2], qsc[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int h = 32 * hh + 16 * nt + c16;
    wv[nt] = a.w[(int64_t)t * kHI + h];
    if (!a.fp8) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qb[nt][ks] = ld16((const uint16_t*)a.qI + ((int64_t)t * kHI + h) * kDI + 32 * ks + 8 * g);
    } else {
      const uint4* p = reinterpret_cast<const uint4*>((const uint8_t*)a.qI + ((int64_t)t * kHI + h) * kDI + 32 * g);
      const uint4 lo = p[0], hi = p[1];
      q8[nt] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      qsc[nt] = a.qI_scale[(int64_t)t * kHI + h];
    }
  }

  // kI block jb: 64 rows of 16-byte chunks, 2 per thread (bf16 rows: the fp8 path reads the
  // dequantized copy), fp8 codes 1 per thread and the row scales; rows past the last visible
  // key repeat row0 (finite; their g is 0)
  uint4 pre[2], pre8;
  float pre_s = 0.f;
  float pre_g[4][4];   // g of keys 16 mt + 4 g + i of the fetched block (0 past nv_w)
  const uint16_t* kI16 = a.fp8 ? a.kI16 : (const uint16_t*)a.kI;
  auto fetch = [&](int jb) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 512 * u, row = e >> 4, ch = e & 15;
      const int key = kKB * jb + row;
      pre[u] = *reinterpret_cast<const uint4*>(kI16 + (int64_t)(row0 + (key < nv_max ? key : 0)) * kDI + 8 * ch);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = kKB * jb + 16 * mt + 4 * g + i;
        pre_g[mt][i] = j < nv_w ? grow[j] : 0.f;
      }
    if (a.fp8) {
      const int row = tid >> 3, ch = tid & 7;
      const int key = kKB * jb + row;
      pre8 = *reinterpret_cast<const uint4*>((const uint8_t*)a.kI + (int64_t)(row0 + (key < nv_max ? key : 0)) * kDI + 16 * ch);
      if (tid < kKB) {
        const int k2 = kKB * jb + tid;
        pre_s = a.kI_scale[row0 + (k2 < nv_max ? k2 : 0)];
      }
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 512 * u, row = e >> 4, ch = e & 15;
      *reinterpret_cast<uint4*>(&KIt[buf][row][8 * ch]) = pre[u];
    }
    if (a.fp8) {
      const int row = tid >> 3, ch = tid & 7;
      *reinterpret_cast<uint4*>(&KI8[buf][row][16 * ch]) = pre8;
      if (tid < kKB) ksc_s[buf][tid] = pre_s;
    }
  };

  f32x4 acc[2][8];   // dqI: heads 32 hh + 16 nt + 4 g + i, d 16 dt + c16
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dwp[2] = {0.f, 0.f};
  const int jr = c16 >> 2, jc = 4 * (c16 & 3);

  if (nblk > 0) {
    fetch(0);
    commit(0);
  }
  for (int jb = 0; jb < nblk; ++jb) {
    const int buf = jb & 1;
    __syncthreads();
    // g of keys 16 mt + 4 g + i of the block for this wave's query (0 past its visible range),
    // fetched with the block
    float gk[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) gk[mt][i] = pre_g[mt][i];
    if (jb + 1 < nblk) fetch(jb + 1);
    // z^T[key 16 mt + 4 g + i][head 32 hh + 16 nt + c16]; E as the A operand of dqI = E kI
    // with k-step ks over key tiles 2 ks (k-slots 8g..8g+3) and 2 ks + 1 (8g+4..8g+7)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // kI^T B operands of this k-step, shared by the 2 head tiles
      bf16x8 kbt[8];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        kbt[dt] = join8(ld_tr(&KIt[buf][32 * ks + 4 * g + jr][16 * dt + jc]),
                        ld_tr(&KIt[buf][32 * ks + 16 + 4 * g + jr][16 * dt + jc]));
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        uint32_t e4[4];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int mt = 2 * ks + h2;
          f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
          if (!a.fp8) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
              z = mfma16(ld16(&KIt[buf][16 * mt + c16][32 * kk + 8 * g]), qb[nt][kk], z);
          } else {
            const uint4* kp = reinterpret_cast<const uint4*>(&KI8[buf][16 * mt + c16][32 * g]);
            const uint4 k0 = kp[0], k1 = kp[1];
            z = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                i32x8{(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w, (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w},
                q8[nt], z, 0, 0, 0, 127, 0, 127);
#pragma unroll
            for (int i = 0; i < 4; ++i) z[i] = z[i] * ksc_s[buf][16 * mt + 4 * g + i] * qsc[nt];
          }
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            dwp[nt] = fmaf(gk[mt][i], fmaxf(z[i], 0.f), dwp[nt]);
            dwp[nt] = fmaf(gk[mt][i + 1], fmaxf(z[i + 1], 0.f), dwp[nt]);
            const float e0 = z[i] > 0.f ? gk[mt][i] * wv[nt] : 0.f;
            const float e1 = z[i + 1] > 0.f ? gk[mt][i + 1] * wv[nt] : 0.f;
            e4[2 * h2 + (i >> 1)] = pack_bf16x2(e0, e1);
          }
        }
        const bf16x8 ea = __builtin_bit_cast(bf16x8, make_uint4(e4[0], e4[1], e4[2], e4[3]));
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[nt][dt] = mfma16(ea, kbt[dt], acc[nt][dt]);
      }
    }
    if (jb + 1 < nblk) commit(buf ^ 1);
  }
  if (!active) return;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float v = dwp[nt];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (g == 0) a.dw[(int64_t)t * kHI + 32 * hh + 16 * nt + c16] = v;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a.dqI[((int64_t)t * kHI + 32 * hh + 16 * nt + 4 * g + i) * kDI + 16 * dt + c16] = acc[nt][dt][i];
  }
}

// bf16 copy of fp8 rows of d_I codes (code * row scale, rounded once): rows row_lo ..
// row_lo + n_rows - 1 (at most *n_max of them when n_max is given) to out[(row - row_lo) d_I]
__global__ __launch_bounds__(256) void k_kld_dequant(const uint8_t* __restrict__ codes,
                                                    const float* __restrict__ scale,
                                                    int64_t row_lo, int64_t n_rows,
                                                    const int32_t* __restrict__ n_max,
                                                    uint16_t* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 8 elements each
  const int64_t rows = n_max ? min(n_rows, (int64_t)*n_max - row_lo) : n_rows;
  if (e >= rows * (kDI / 8)) return;
  const int64_t src = row_lo * kDI + 8 * e;
  const uint2 c = *reinterpret_cast<const uint2*>(codes + src);
  const float s = scale[src / kDI];
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t wd = i < 2 ? c.x : c.y;
    const uint32_t b0 = (wd >> (16 * (i & 1))) & 0xffu, b1 = (wd >> (16 * (i & 1) + 8)) & 0xffu;
    o[i] = (uint32_t)f32_to_bf16_bits(e4m3_to_f32(b0) * s) |
           ((uint32_t)f32_to_bf16_bits(e4m3_to_f32(b1) * s) << 16);
  }
  *reinterpret_cast<uint4*>(out + 8 * e) = make_uint4(o[0], o[1], o[2], o[3]);
}

static bool kld_handles(const Shape& sh) {
  return sh.teacher == 2 && sh.mode == 0 && sh.dtype == 1 && sh.H == kH && sh.D == kD &&
         sh.HI == kHI && sh.dI == kDI && sh.idx_dtype != 0 &&
         sh.max_seqlen / sh.r <= kKB * kMaxBlocks;
}

static int kld_rows(const Shape& sh) { return sh.T < kChunkRows ? sh.T : kChunkRows; }

bool indexer_kl_recomputes_scores(const Shape& sh) { return kld_handles(sh); }

size_t indexer_kl_dense_workspace(const Shape& sh) {
  if (!kld_handles(sh) || sh.T == 0) return 0;
  const size_t rows = (size_t)kld_rows(sh);
  size_t bytes = rows * (size_t)(sh.max_seqlen / sh.r) * sizeof(float);
  bytes = (bytes + 255) & ~(size_t)255;
  if (sh.idx_dtype == 2)
    bytes += rows * kHI * kDI * sizeof(uint16_t) + (size_t)(sh.T / sh.r) * kDI * sizeof(uint16_t);
  return bytes;
}

hipError_t launch_indexer_kl_dense(const Shape& sh, const KlIO& io, hipStream_t s,
                                   bool* handled) {
  *handled = false;
  if (!kld_handles(sh)) return hipSuccess;
  *handled = true;
  const int n_cap = sh.max_seqlen / sh.r;
  const int rows = kld_rows(sh);
  KldArgs a;
  a.q = (const uint16_t*)io.q;
  a.kv_cmp = (const uint16_t*)io.kv_cmp;
  a.scores = io.scores;
  a.ld = io.ld;
  a.s_t0 = 0;
  a.qI = io.qI;
  a.qI_scale = io.qI_scale;
  a.w = io.w;
  a.kI = io.kI;
  a.kI_scale = io.kI_scale;
  a.cu = sh.cu;
  a.cu_cmp = sh.cu_cmp;
  a.g = (float*)io.ws;
  size_t g_bytes = (size_t)rows * n_cap * sizeof(float);
  g_bytes = (g_bytes + 255) & ~(size_t)255;
  uint16_t* q16 = sh.idx_dtype == 2 ? (uint16_t*)((char*)io.ws + g_bytes) : nullptr;
  uint16_t* k16 = sh.idx_dtype == 2 ? q16 + (size_t)rows * kHI * kDI : nullptr;
  a.kI16 = k16;
  a.qI16 = sh.idx_dtype == 2 ? q16 : (const uint16_t*)io.qI;
  a.q16_t0 = 0;
  a.kl = io.kl;
  a.dkI = io.dkI;
  a.gs = io.grad_scale;
  a.scale_log2 = sh.scale * 1.44269504088896341f;
  a.B = sh.B;
  a.T = sh.T;
  a.r = sh.r;
  a.n_cap = n_cap;
  a.tc_blocks = (sh.T / sh.r + 4 * kKB - 1) / (4 * kKB);   // 256-row key groups
  a.fp8 = sh.idx_dtype == 2;
  const bool grads = io.dqI != nullptr;
  if (grads && a.fp8) {
    const int64_t n = (int64_t)(sh.T / sh.r) * (kDI / 8);
    hipLaunchKernelGGL(k_kld_dequant, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const uint8_t*)io.kI, io.kI_scale, (int64_t)0, (int64_t)(sh.T / sh.r),
                       sh.cu_cmp + sh.B, k16);
  }
  for (int t_lo = 0; t_lo < sh.T; t_lo += rows) {
    a.t_lo = t_lo;
    a.t_hi = t_lo + rows < sh.T ? t_lo + rows : sh.T;
    if (!io.scores) {
      // no score matrix given: the chunk's student scores are formed into its rows of the
      // workspace (row t - t_lo), which the teacher pass then overwrites with g in place
      bool sc_handled = false;
      hipError_t e = launch_index_scores_mfma(sh, io.qI, io.qI_scale, io.w, io.kI, io.kI_scale,
                                              a.g, n_cap, s, &sc_handled, a.t_lo, a.t_hi);
      if (e != hipSuccess) return e;
      if (!sc_handled) return hipErrorInvalidValue;
      a.scores = a.g;
      a.ld = n_cap;
      a.s_t0 = a.t_lo;
    }
    hipLaunchKernelGGL(k_kld_teacher, dim3(kChunkRows / 4 + sh.B), dim3(512), 0, s, a);
    if (!grads) continue;
    a.dqI = io.dqI;
    a.dw = io.dw;
    hipLaunchKernelGGL(k_kld_queries, dim3(kChunkRows / 4 + sh.B), dim3(512), 0, s, a);
    if (a.fp8) {
      const int64_t n = (int64_t)(a.t_hi - a.t_lo) * kHI * (kDI / 8);
      hipLaunchKernelGGL(k_kld_dequant, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                         (const uint8_t*)io.qI, io.qI_scale, (int64_t)a.t_lo * kHI,
                         (int64_t)(a.t_hi - a.t_lo) * kHI, (const int32_t*)nullptr, q16);
      a.q16_t0 = a.t_lo;   // the copy holds rows t - t_lo
    }
    hipLaunchKernelGGL(k_kld_keys, dim3(a.tc_blocks + sh.B, kChunkRows / kRange), dim3(512), 0,
                       s, a);
  }
  return hipGetLastError();
}

}  // namespace csa
