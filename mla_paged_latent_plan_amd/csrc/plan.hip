// mla_decode_plan kernel: split-KV work plan computed on the device from the sequence lengths.
//
// The pages only say that a metadata step produces "tile scheduling metadata and split
// information" (FlashMLA wrapper, get_mla_metadata) and that a per-forward plan with a work list
// feeds the attention (HALOps, mla_attention_plan); the algorithm is this library's own:
//   n_g    effective rows of query group g (all rows / window union / index-list length)
//   nblk_g ceil(n_g / 64);  cost_g = nblk_g + FIXED (0 if no blocks);  P_g = exclusive prefix
//   quota  max(1, ceil(sum cost / U))
//   block k of group g sits at position P_g + FIXED + k and goes to unit min(U-1, pos / quota);
//   a split is a maximal run of a group's blocks in one unit.
// One workgroup of 1024 threads: two block-wide prefix scans (cost, then split counts), then the
// split records and the per-unit pointers are written in parallel. Integer arithmetic only, so
// the result is reproducible bit for bit.
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kPlanThreads = 1024;

__device__ __forceinline__ long long block_exclusive_scan(long long v, long long* s_warp,
                                                          long long* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  long long x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    long long t = __shfl_up(x, off, 64);
    if (lane >= off) x += t;
  }
  if (lane == 63) s_warp[w] = x;
  __syncthreads();
  if (w == 0) {
    long long y = (lane < kPlanThreads / 64) ? s_warp[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      long long t = __shfl_up(y, off, 64);
      if (lane >= off) y += t;
    }
    if (lane < kPlanThreads / 64) s_warp[lane] = y;
  }
  __syncthreads();
  long long before = (w > 0) ? s_warp[w - 1] : 0;
  *total = s_warp[kPlanThreads / 64 - 1];
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ long long s_P[kMaxGroups];   // exclusive prefix of cost
  __shared__ int s_nblk[kMaxGroups];
  __shared__ long long s_warp[kPlanThreads / 64];
  const int tid = threadIdx.x;
  const int G = a.G, U = a.U, FIXED = a.fixed;
  int32_t* plan = a.plan;
  const PlanLayout& lay = a.lay;
  const int per = (G + kPlanThreads - 1) / kPlanThreads;
  const int g_begin = min(G, tid * per), g_end = min(G, g_begin + per);

  // 1. effective rows, blocks, local cost sums
  long long my_cost = 0;
  for (int g = g_begin; g < g_end; ++g) {
    int j0 = 0, n = 0;
    if (a.topk > 0) {
      const int b = g / a.Sq;
      const int L = a.seqlens[b];
      if (L > 0) {
        n = a.topk;
        if (a.topk_lens != nullptr) n = min(max(a.topk_lens[g], 0), a.topk);
      }
    } else {
      const int L = a.seqlens[g];
      if (L > 0) {
        if (a.window > 0) {
          n = (int)min((long long)L, (long long)a.window + a.Sq - 1);
          j0 = L - n;
        } else {
          n = L;
        }
      }
    }
    plan[lay.grp_rows + 2 * g] = j0;
    plan[lay.grp_rows + 2 * g + 1] = n;
    const int nb = (n + kBlockRows - 1) / kBlockRows;
    s_nblk[g] = nb;
    my_cost += nb > 0 ? (long long)nb + FIXED : 0;
  }
  long long total = 0;
  long long pre = block_exclusive_scan(my_cost, s_warp, &total);
  for (int g = g_begin; g < g_end; ++g) {
    s_P[g] = pre;
    const int nb = s_nblk[g];
    pre += nb > 0 ? (long long)nb + FIXED : 0;
  }
  const long long quota = max(1LL, (total + U - 1) / U);

  // 2. split counts per group and their prefix (grp_ptr)
  long long my_ns = 0;
  for (int g = g_begin; g < g_end; ++g) {
    const int nb = s_nblk[g];
    if (nb > 0) {
      const long long p0 = s_P[g] + FIXED;
      const long long uf = min((long long)U - 1, p0 / quota);
      const long long ul = min((long long)U - 1, (p0 + nb - 1) / quota);
      my_ns += ul - uf + 1;
    }
  }
  long long S = 0;
  long long sp = block_exclusive_scan(my_ns, s_warp, &S);

  // 3. split records
  for (int g = g_begin; g < g_end; ++g) {
    plan[lay.grp_ptr + g] = (int32_t)sp;
    const int nb = s_nblk[g];
    if (nb > 0) {
      const long long p0 = s_P[g] + FIXED;
      const long long uf = min((long long)U - 1, p0 / quota);
      const long long ul = min((long long)U - 1, (p0 + nb - 1) / quota);
      for (long long u = uf; u <= ul; ++u) {
        const long long kb = (u == uf) ? 0 : u * quota - p0;
        const long long ke = (u == ul) ? nb : (u + 1) * quota - p0;
        int32_t* rec = plan + lay.splits + 4 * sp;
        rec[0] = g;
        rec[1] = (int32_t)kb;
        rec[2] = (int32_t)ke;
        rec[3] = (int32_t)u;
        // the split's descriptor: group, request, first row, rows, request length, step range
        // (32-row steps holding at least one row), the group's split count
        const int j0 = plan[lay.grp_rows + 2 * g], n = plan[lay.grp_rows + 2 * g + 1];
        const int b = (a.topk > 0) ? g / a.Sq : g;
        int4* d = reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(plan) + lay.sdesc_bytes_off) + 2 * sp;
        d[0] = make_int4(g, b, j0, n);
        d[1] = make_int4(a.seqlens[b], 2 * (int)kb, min(2 * (int)ke, (n + 31) / 32), (int)(ul - uf + 1));
        ++sp;
      }
    }
  }
  if (tid == 0) {
    plan[lay.grp_ptr + G] = (int32_t)S;
    int32_t* h = plan;
    h[H_MAGIC] = kPlanMagic;
    h[H_G] = G;
    h[H_U] = U;
    h[H_S] = (int32_t)S;
    h[H_R] = a.R;
    h[H_MTILES] = a.m_tiles;
    h[H_MTILE] = a.m_tile;
    h[H_QUOTA] = (int32_t)quota;
    h[H_FIXED] = FIXED;
    h[H_TOTAL] = (int32_t)total;
    h[H_SMAX] = G + U;
    for (int i = H_SMAX + 1; i < kHeaderWords; ++i) h[i] = 0;
  }
  // zero row used as the source of masked rows
  uint32_t* zr = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(plan) + lay.zero_row_bytes_off);
  for (int i = tid; i < kZeroRowBytes / 4; i += kPlanThreads) zr[i] = 0u;
  __syncthreads();  // split records visible to the whole workgroup

  // 4. unit_ptr[u] = number of splits with unit < u
  const int32_t* rec = plan + lay.splits;
  if (S == 0) {
    for (int u = tid; u <= U; u += kPlanThreads) plan[lay.unit_ptr + u] = 0;
  } else {
    const int u0 = rec[3];
    for (int u = tid; u <= u0; u += kPlanThreads) plan[lay.unit_ptr + u] = 0;
    for (long long s = tid; s < S; s += kPlanThreads) {
      const int us = rec[4 * s + 3];
      const int un = (s + 1 < S) ? rec[4 * (s + 1) + 3] : U;
      for (int u = us + 1; u <= un; ++u) plan[lay.unit_ptr + u] = (int32_t)(s + 1);
    }
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
