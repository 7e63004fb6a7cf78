// mla_plan.hip -- split plan for MLA decode: which stretch of the paged KV each
// persistent workgroup handles.
//
// The pages of all requests are laid end to end.  Each request costs its page
// count plus a fixed per-request cost (loading its queries and writing its
// output), and the concatenation is cut into nwg stretches of equal cost.  A
// stretch boundary that falls inside a request splits it; the pieces are merged
// by their LSE afterwards.  This follows the scheduling metadata of the FlashMLA
// paragraph of "MLA inference: two computation paths and FlashMLA" (computed once
// from the context lengths, deciding which stretch of KV each compute unit
// handles) and the FlashMLA guide's "Native Ragged Sequence Batching" (work
// assigned by context length so long and short requests share the GPU).
//
// One workgroup of 256 threads does the whole plan on the device from the
// device-resident sequence lengths, so no host synchronisation is needed.  All
// working arrays live in LDS (batch <= kMaxBatch, stretches <= kMaxStretches),
// so every binary search is a handful of LDS reads.
#include <hip/hip_runtime.h>

#define MLA_HD __host__ __device__
#include "mla_launch.h"
#include "mla_workspace.h"

namespace mla {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / 64;

// Inclusive scan over the workgroup; `wsum` is scratch for the per-wave totals.
// Returns the inclusive prefix of this thread; *total receives the block total.
// Two independent values are scanned together (one set of barriers).
__device__ int2 block_scan2(int2 v, int2* wsum, int2* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int yx = __shfl_up(v.x, off, 64), yy = __shfl_up(v.y, off, 64);
    if (lane >= off) {
      v.x += yx;
      v.y += yy;
    }
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  int2 pre = make_int2(0, 0), tot = make_int2(0, 0);
#pragma unroll
  for (int i = 0; i < kPlanWaves; i++) {   // a handful of waves: read the totals directly
    const int2 x = wsum[i];
    if (i < w) {
      pre.x += x.x;
      pre.y += x.y;
    }
    tot.x += x.x;
    tot.y += x.y;
  }
  *total = tot;
  __syncthreads();
  return make_int2(v.x + pre.x, v.y + pre.y);
}
__device__ int block_scan(int v, int2* wsum, int* total) {
  int2 t;
  const int2 r = block_scan2(make_int2(v, 0), wsum, &t);
  *total = t.x;
  return r.x;
}

// Largest index i in [0, n) with key(i) <= x, or -1.
template <typename F>
__device__ int last_le(int n, int x, F key) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (key(mid) <= x) lo = mid + 1; else hi = mid;
  }
  return lo - 1;
}

__global__ __launch_bounds__(kPlanThreads) void mla_plan_kernel(const int32_t* __restrict__ seqlens, char* ws,
                                                                Layout lay, int batch, int seqlen_q, int rows,
                                                                int nwg, int max_blocks) {
  __shared__ int s_cost[kMaxBatch + 1];   // exclusive prefix of per-request cost
  __shared__ int s_first[kMaxBatch];      // first page (global position) of each request
  __shared__ int s_np[kMaxBatch];         // pages of each request
  __shared__ int s_bnd[kMaxStretches + 1];   // stretch boundaries in page positions
  __shared__ int s_ne[kMaxStretches + 1];    // non-empty stretches before each stretch
  __shared__ int2 wsum[kPlanWaves];
  __shared__ unsigned flags;

  Header* hdr = reinterpret_cast<Header*>(ws + lay.header);
  WgInfo* wgi = reinterpret_cast<WgInfo*>(ws + lay.wg_info);
  ReqInfo* req = reinterpret_cast<ReqInfo*>(ws + lay.req_info);
  const int t = threadIdx.x;
  const int max_len = max_blocks * kPageSize;
  if (t == 0) flags = 0;
  __syncthreads();

  // 1. pages and cost per request; exclusive prefix sums of both.
  int carry_p = 0, carry_c = 0;
  for (int base = 0; base < batch; base += kPlanThreads) {
    const int b = base + t;
    int L = 0;
    if (b < batch) {
      L = seqlens[b];
      if (L < seqlen_q || L > max_len) atomicOr(&flags, 1u);
      L = L < 0 ? 0 : (L > max_len ? max_len : L);
    }
    const int np = (L + kPageSize - 1) / kPageSize;
    const int cost = np > 0 ? np + kPlanCostPerRequest : 0;
    int2 tot;
    const int2 inc = block_scan2(make_int2(np, cost), wsum, &tot);
    const int inc_p = inc.x, inc_c = inc.y, tot_p = tot.x, tot_c = tot.y;
    if (b < batch) {
      s_first[b] = carry_p + inc_p - np;
      s_np[b] = np;
      s_cost[b] = carry_c + inc_c - cost;
      req[b].seqlen = L;
    }
    carry_p += tot_p;
    carry_c += tot_c;
  }
  const int total_pages = carry_p;
  const int total_cost = carry_c;
  if (t == 0) s_cost[batch] = total_cost;
  __syncthreads();

  // 2. stretch boundaries in page positions: boundary s sits at cost s * T / nwg;
  //    a boundary inside a request's fixed-cost part moves to its first page.
  for (int s = t; s <= nwg; s += kPlanThreads) {
    int bnd;
    if (s == nwg) {
      bnd = total_pages;
    } else {
      const int x = (int)((int64_t)s * total_cost / nwg);
      const int b = last_le(batch, x, [&](int i) { return s_cost[i]; });
      const int off = x - s_cost[b] - kPlanCostPerRequest;
      bnd = s_first[b] + (off < 0 ? 0 : (off > s_np[b] ? s_np[b] : off));
    }
    s_bnd[s] = bnd;
  }
  __syncthreads();

  // 3. non-empty stretches: exclusive prefix count, then per-stretch info.
  {
    int carry = 0;
    for (int base = 0; base <= nwg; base += kPlanThreads) {
      const int s = base + t;
      const int ne = (s < nwg && s_bnd[s + 1] > s_bnd[s]) ? 1 : 0;
      int tot;
      const int inc = block_scan(ne, wsum, &tot);
      if (s <= nwg) s_ne[s] = carry + inc - ne;
      carry += tot;
    }
  }
  __syncthreads();
  for (int s = t; s < nwg; s += kPlanThreads) {
    WgInfo w;
    w.page_begin = s_bnd[s];
    w.page_end = s_bnd[s + 1];
    w.b_begin = w.page_begin < total_pages ? last_le(batch, w.page_begin, [&](int i) { return s_first[i]; }) : batch;
    w.ne_prefix = s_ne[s];
    wgi[s] = w;
  }

  // 4. per request: how many stretches hold it, and its partial slots.
  int carry = 0;
  for (int base = 0; base < batch; base += kPlanThreads) {
    const int b = base + t;
    int nsplit = 0, ne_lo = 0;
    if (b < batch && s_np[b] > 0) {
      const int first = s_first[b], end = first + s_np[b];
      // first stretch whose end is past the request's first page
      const int s_lo = 1 + last_le(nwg, first, [&](int i) { return s_bnd[i + 1]; });
      // last stretch whose begin is before the request's end
      const int s_hi = last_le(nwg, end - 1, [&](int i) { return s_bnd[i]; });
      nsplit = s_ne[s_hi + 1] - s_ne[s_lo];
      ne_lo = s_ne[s_lo];
    }
    const int slots = nsplit > 1 ? nsplit : 0;
    int tot;
    const int inc = block_scan(slots, wsum, &tot);
    if (b < batch) {
      ReqInfo r;
      r.page_first = s_first[b];
      r.npages = s_np[b];
      r.nsplit = nsplit;
      r.slot_off = carry + inc - slots;
      r.ne_lo = ne_lo;
      r.seqlen = req[b].seqlen;
      r.pad0 = r.pad1 = 0;
      req[b] = r;
    }
    carry += tot;
  }
  if (t == 0) {
    Header h;
    h.magic = kMagic;
    h.flags = flags;
    h.batch = batch;
    h.rows = rows;
    h.nwg = nwg;
    h.nrb = row_blocks(rows);
    h.max_slots = 2 * nwg;
    h.total_pages = total_pages;
    h.used_slots = carry;
    for (int i = 0; i < 7; i++) h.pad[i] = 0;
    *hdr = h;
  }
}

}  // namespace

hipError_t launch_plan(const int32_t* seqlens, void* ws, const Layout& lay, int batch, int seqlen_q, int rows,
                       int nwg, int max_blocks, hipStream_t stream) {
  void* args[] = {(void*)&seqlens, (void*)&ws, (void*)&lay, (void*)&batch, (void*)&seqlen_q,
                  (void*)&rows, (void*)&nwg, (void*)&max_blocks};
  return hipLaunchKernel((const void*)mla_plan_kernel, dim3(1), dim3(kPlanThreads), args, 0, stream);
}

}  // namespace mla
