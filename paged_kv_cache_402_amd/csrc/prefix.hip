// Shared-prefix pass of decode attention on gfx950 matrix cores.
//
// When many sequences list the same physical blocks for their leading partitions (one
// system prompt shared by a whole batch: P1 §6.1, P3 §2.2.3 and §2.2.8), the per-sequence
// pass would read those blocks and redo the same exponentials and products once per
// sequence. Here one workgroup takes one KV head, one shared partition and 64 query rows of
// the group at once (16 rows per wave: 16 / G sequences x G query heads), so the products
// become dense matrix products:
//   S^T (16 tokens x 16 rows) = K (16 tokens x d) . Q^T (d x 16 rows)     [v_mfma 16x16x32]
//   O^T (16 cols x 16 rows)  += V^T (16 cols x 32 tokens) . P^T (32 tokens x 16 rows)
// and it writes the same (max, exponent sum, accumulator) partials as the per-partition
// kernel, which the partition merge then combines with the sequences' own partitions.
//
// Operand layouts of v_mfma_f32_16x16x32_{bf16,f16}: lane l supplies A[l % 16][8g .. 8g+8)
// and B[8g .. 8g+8)[l % 16], g = l / 16, and receives C[4g + i][l % 16], i = 0..3.
// With S^T as C, lane l holds the scores of its own row r = l % 16 for the tokens
// 4g + i and 16 + 4g + i of a 32-token step. The P^T operand of the value product takes those
// eight values as they lie: the contraction index 8g + e stands for token 4g + e (e < 4) or
// 16 + 4g + e - 4 (e >= 4), and V^T is read from LDS in that same token order. O^T as C
// gives lane l its own row's accumulators for columns 16t + 4g + i, so rescaling a row by
// its new maximum needs no data movement.
//
// Softmax weights p are fp32; the value product takes them as two 16-bit operands, p = hi +
// lo with hi = p truncated to 16 bits and lo = (p - hi) truncated, so the weights keep about
// 15 significant bits with bf16 and 21 with fp16 (a single bf16 p would err by up to 2^-8
// relative per weight).
//
// The pass is bound by VALU issue (two waves per SIMD), so the per-step arithmetic is kept
// short: the weights use a reference max that moves only when a row's max passes it by more
// than 8 (log2 units), so the accumulators, which live in the matrix-core registers, are
// rescaled rarely instead of every step (weights then reach 2^8, which fp32 sums and the
// 16-bit halves carry with the same relative precision); v_exp_f32 directly; the row max
// over the four lanes of a row through lane swaps instead of LDS shuffles.

#include <math.h>

#include "common.h"
#include "launch.h"

namespace pkv {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <int DT> __device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c);
template <> __device__ __forceinline__ f32x4 mma<BF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mma<F16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// (p0, p1) -> packed 16-bit halves hi = (hi0, hi1) and lo = (lo0, lo1) with p ~= hi + lo:
// hi is p truncated, lo the exact fp32 remainder p - hi, truncated in turn.
template <int DT> __device__ __forceinline__ void split_pair(float p0, float p1, uint32_t& hi,
                                                            uint32_t& lo);
template <>
__device__ __forceinline__ void split_pair<BF16>(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  const uint32_t h0 = as_u32(p0) & 0xFFFF0000u, h1 = as_u32(p1) & 0xFFFF0000u;
  hi = __builtin_amdgcn_perm(h1, h0, 0x07060302u);        // upper halves of h0, h1
  lo = __builtin_amdgcn_perm(as_u32(p1 - as_f32(h1)), as_u32(p0 - as_f32(h0)), 0x07060302u);
}
template <>
__device__ __forceinline__ void split_pair<F16>(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(p0, p1);      // round toward zero
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(p0 - (float)h[0], p1 - (float)h[1]));
}

// max over lanes l, l ^ 16, l ^ 32 and l ^ 48: each swap leaves every lane with its own and its
// partner's value in the two results
__device__ __forceinline__ float row4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
  x = fmaxf(x, fmaxf(as_f32(a[0]), as_f32(a[1])));
  const auto b = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  return fmaxf(x, fmaxf(as_f32(b[0]), as_f32(b[1])));
}

constexpr float kRescaleSlack = 8.f;      // log2 units a row's max may pass its reference

constexpr int kD = kPrefixHeadDim;        // head_dim of this pass
constexpr int kRow = kD * 2;              // bytes of one token row of one head
constexpr int kVtStride = 32 * 2 + 8;     // bytes of one V^T row in LDS (32 tokens + pad)
constexpr int kKStride = kRow + 16;       // bytes of one K row in LDS (padded)
constexpr int kMaxIds = kPrefixMaxIds;    // block ids of one partition kept in LDS

}  // namespace

// PF: steps of loads in flight ahead of the math; it divides part / 32.
template <int DT, int G, int PF>
__global__ __launch_bounds__(256) void paged_prefix_kernel(PrefixArgs a) {
  constexpr int SPW = 16 / G;             // sequences per wave
  constexpr int SPG = 4 * SPW;            // sequences per workgroup
  constexpr int NJ = kD / 32;             // d-slices of the score product
  constexpr int NT = kD / 16;             // column tiles of the value product
  __shared__ int s_ids[kMaxIds];
  __shared__ __align__(16) unsigned char s_vt[2][kD * kVtStride];
  __shared__ __align__(16) unsigned char s_k[2][32 * kKStride];

  const int kvh = blockIdx.x % a.num_kv_heads;
  const int chunk = blockIdx.x / a.num_kv_heads;
  const int p = blockIdx.y;                           // shared partition
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int r = lane & 15;

  // ---- this lane's query row: member mi, query head h ----
  // members naming a sequence outside the batch are skipped (their rows read and write
  // nothing); a first member outside the batch leaves the whole pass without a block list
  const int rep = a.members[0];
  if ((unsigned)rep >= (unsigned)a.num_seqs) return;
  const int mi = chunk * SPG + wave * SPW + r / G;
  const int bm = mi < a.num_members ? a.members[mi] : -1;
  const bool valid = (unsigned)bm < (unsigned)a.num_seqs;
  const int b = valid ? bm : 0;
  const int h = kvh * G + (r % G);
  u32x4 qv[NJ];
  {
    const unsigned char* qrow =
        (const unsigned char*)a.q + ((size_t)b * a.num_q_heads + h) * kRow;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      qv[j] = valid ? load16(qrow + (32 * j + 8 * g) * 2) : u32x4{0u, 0u, 0u, 0u};
  }

  // ---- the member's length, clamped as the per-partition kernel clamps it: the row attends
  // only to tokens before it, so a member that ends inside a shared partition still gets
  // exact partials (and its output row, when it has one partition only) ----
  const int cap = a.max_blocks << a.bs_log2;
  int Lr = valid ? a.seq_lens[b] : 0;
  Lr = Lr < 0 ? 0 : (Lr > cap ? cap : Lr);
  const int nrow = Lr - p * a.part;        // tokens of this partition the row attends to

  // ---- the partition's block ids (from the first member's table); an entry outside the
  // pool is kept as -1: its tokens are left out (as the per-partition kernel leaves them
  // out), and its loads read block 0, which is inside the pool ----
  const int nblk = a.part >> a.bs_log2;
  const int32_t* trow = a.block_tables + (size_t)rep * a.max_blocks +
                        (((size_t)p * a.part) >> a.bs_log2);
  int bad = 0;
  for (int i = tid; i < nblk; i += 256) {
    const int id = trow[i];
    const bool in_pool = (unsigned)id < (unsigned)a.num_blocks;
    s_ids[i] = in_pool ? id : -1;
    bad |= !in_pool;
  }
  const bool any_bad = __syncthreads_or(bad) != 0;
  // per-token masking only in waves that need it (the usual shared prefix needs none)
  const bool need_mask = any_bad || __builtin_amdgcn_ballot_w64(nrow < a.part) != 0;

  const int bs_mask = (1 << a.bs_log2) - 1;
  const size_t head_bytes = (size_t)kRow << a.bs_log2;       // one (block, head) tile
  const size_t block_bytes = head_bytes * a.num_kv_heads;
  const unsigned char* kbase = (const unsigned char*)a.k_cache + kvh * head_bytes;
  const unsigned char* vbase = (const unsigned char*)a.v_cache + kvh * head_bytes;
  auto row_off = [&](int tok) -> size_t {                     // partition-relative token
    const int blk = max(s_ids[tok >> a.bs_log2], 0);
    return (size_t)blk * block_bytes + (size_t)(tok & bs_mask) * kRow;
  };

  // Staging of one 32-token step, shared by the four waves: thread -> token pair tid % 16,
  // columns 8 (tid / 16) .. +8 of K and of V (four 16-byte loads). K goes to LDS row-major
  // (rows padded to 272 bytes), V transposed; with this mapping the 32 lanes of one LDS cycle
  // write the transposed V tile to 32 different banks (token pairs 0..15 of two column groups).
  const int vp = tid & 15;
  const int vc = tid >> 4;
  // default cache policy (not the non-temporal one of the per-partition pass): the other row
  // chunks of this (KV head, partition) read the same rows, from L2
  auto load_step = [&](int step, u32x4 (&x)[4]) {
    const int tok = step * 32 + 2 * vp;                   // even: tok + 1 is in the same block
    const size_t o0 = row_off(tok) + 16 * vc, o1 = o0 + kRow;
    x[0] = load16(kbase + o0);
    x[1] = load16(kbase + o1);
    x[2] = load16(vbase + o0);
    x[3] = load16(vbase + o1);
  };
  auto store_step = [&](int buf, const u32x4 (&x)[4]) {
    unsigned char* kd = s_k[buf] + (size_t)(2 * vp) * kKStride + 16 * vc;
    store16(kd, x[0]);
    store16(kd + kKStride, x[1]);
    unsigned char* dst = s_vt[buf] + (size_t)(8 * vc) * kVtStride + 4 * vp;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // element e of token tok and of token tok + 1, packed: one byte permute
      const uint32_t w0 = x[2][e >> 1], w1 = x[3][e >> 1];
      *reinterpret_cast<uint32_t*>(dst + e * kVtStride) =
          __builtin_amdgcn_perm(w1, w0, (e & 1) ? 0x07060302u : 0x05040100u);
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one step (the step-th 32 tokens of the partition) of math on the staged tiles of buffer buf
  auto compute = [&](int buf, int step) {
    // every LDS operand of the step first (K: 8 x 16 B, V^T: 16 x 8 B), so their latencies
    // overlap one another and the products instead of being paid one read at a time
    const unsigned char* kt = s_k[buf] + (size_t)r * kKStride + 16 * g;
    const unsigned char* vt = s_vt[buf] + (size_t)r * kVtStride + 8 * g;
    u32x4 ka[2][NJ];
    u32x4 av[NT];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int j = 0; j < NJ; ++j) ka[hh][j] = load16(kt + (size_t)(16 * hh) * kKStride + 64 * j);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // V^T rows 16 t + r, tokens 4 g .. 4 g + 3 and 16 + 4 g .. + 3
      const unsigned char* row = vt + (size_t)(16 * t) * kVtStride;
      const uint2 x0 = *reinterpret_cast<const uint2*>(row);
      const uint2 x1 = *reinterpret_cast<const uint2*>(row + 32);
      av[t] = u32x4{x0.x, x0.y, x1.x, x1.y};
    }
    __builtin_amdgcn_sched_barrier(0);
    // scores of the 32 tokens for this lane's row (log2 units); K rows 16 hh + r
    float sc[8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NJ; ++j) c = mma<DT>(ka[hh][j], qv[j], c);
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * hh + i] = c[i] * a.scale_log2;
    }
    if (need_mask) {
      // tokens 16 hh + 4 g + i of the step: the four share one block (blocks hold >= 8)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int tok = step * 32 + 16 * hh + 4 * g;
        const bool blk_ok = !any_bad || s_ids[tok >> a.bs_log2] >= 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sc[4 * hh + i] = blk_ok && tok + i < nrow ? sc[4 * hh + i] : -INFINITY;
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
    mx = row4_max(mx);
    // move the reference max of the rows whose max passed it by more than the slack (all rows
    // at the first step), rescaling what they have summed so far
    const bool move = mx > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      const float m_new = move ? mx : m_run;
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] *= alpha;
    }
    uint32_t ph[4], pl[4];
    float psum = 0.f;
    // the reference is -inf only while every token of the row so far was left out; then
    // every score is -inf too, and a base of 0 gives them weight 0
    const float mref = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      // sc - m_run <= 8: the weights stay below 2^8; those under 2^-126 flush to zero
      const float p0 = __builtin_amdgcn_exp2f(sc[e] - mref);
      const float p1 = __builtin_amdgcn_exp2f(sc[e + 1] - mref);
      psum += p0 + p1;
      split_pair<DT>(p0, p1, ph[e >> 1], pl[e >> 1]);
    }
    l_run += psum;
    const u32x4 bhi = u32x4{ph[0], ph[1], ph[2], ph[3]};
    const u32x4 blo = u32x4{pl[0], pl[1], pl[2], pl[3]};
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = mma<DT>(av[t], blo, mma<DT>(av[t], bhi, acc[t]));
  };

  // Loads run kPf steps ahead of the math through a ring of registers; the LDS tiles are
  // double-buffered, one barrier per step (a buffer is refilled two steps after its reads,
  // and every wave has passed the barrier in between).
  // PF divides the step count, so the loop body has no branch: the compiler counts the loads
  // in flight exactly and waits only for the oldest step's. Past the last step the loads
  // fetch the last step again.
  const int steps = a.part >> 5;
  u32x4 ring[PF][4];
#pragma unroll
  for (int u = 0; u < PF; ++u) load_step(min(u, steps - 1), ring[u]);
  for (int s0 = 0; s0 < steps; s0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int s = s0 + u;
      store_step(s & 1, ring[u]);
      load_step(min(s + PF, steps - 1), ring[u]);
      __syncthreads();
      compute(s & 1, s);
    }
  }

  const float l_row = xor_sum_from<16>(l_run);
  if (!valid) return;
  const int nparts = Lr == 0 ? 1 : (Lr + a.part - 1) / a.part;
  if (p >= nparts) return;                 // past the member's end: the merge never reads it
  if (nparts == 1) {
    // the member fits this (first) partition: no merge runs for it, so its row is final here
    // (a member of length 0 gets a zero row)
    const size_t o = ((size_t)b * a.num_q_heads + h) * kD + 4 * g;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store_out(a.out, o + 16 * t + i, l_row > 0.f ? acc[t][i] / l_row : 0.f, a.out_dtype);
    return;
  }
  const size_t slot = ((size_t)b * a.num_q_heads + h) * a.pmax + p;
  float* dst = a.ws_acc + slot * kD + 4 * g;
#pragma unroll
  for (int t = 0; t < NT; ++t)
    *reinterpret_cast<float4*>(dst + 16 * t) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
  if (g == 0) {
    a.ws_ml[slot * 2] = m_run;
    a.ws_ml[slot * 2 + 1] = l_row;
  }
}


template <int DT, int G>
static void launch_pf(const PrefixArgs& a, dim3 grid, hipStream_t stream) {
  // two steps of loads in flight measured best (four hold more registers for no gain)
  const int steps = a.part >> 5;
  if (steps % 2 == 0)
    hipLaunchKernelGGL((paged_prefix_kernel<DT, G, 2>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((paged_prefix_kernel<DT, G, 1>), grid, dim3(256), 0, stream, a);
}

template <int DT>
static hipError_t launch_g(const PrefixArgs& a, int group, hipStream_t stream) {
  const int per = prefix_chunk_seqs(group);
  const dim3 grid((unsigned)a.num_kv_heads * ((a.num_members + per - 1) / per),
                  (unsigned)a.prefix_parts);
  switch (group) {
    case 1: launch_pf<DT, 1>(a, grid, stream); break;
    case 2: launch_pf<DT, 2>(a, grid, stream); break;
    case 4: launch_pf<DT, 4>(a, grid, stream); break;
    default: launch_pf<DT, 8>(a, grid, stream); break;
  }
  return hipGetLastError();
}

hipError_t launch_prefix(const PrefixArgs& a, int kv_dtype, int group, hipStream_t stream) {
  return kv_dtype == BF16 ? launch_g<BF16>(a, group, stream) : launch_g<F16>(a, group, stream);
}

}  // namespace pkv
