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
// One workgroup of 1024 threads does the whole plan on the device from the
// device-resident sequence lengths, so no host synchronisation is needed.
#include <hip/hip_runtime.h>

#define MLA_HD __host__ __device__
#include "mla_workspace.h"
#include "mla_launch.h"

namespace mla {
namespace {

constexpr int kPlanThreads = 1024;

// Inclusive scan of one value per thread across the workgroup.
__device__ int64_t block_inclusive_scan(int64_t v, int64_t* tmp) {
  const int t = threadIdx.x;
  tmp[t] = v;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int64_t add = t >= off ? tmp[t - off] : 0;
    __syncthreads();
    tmp[t] += add;
    __syncthreads();
  }
  const int64_t r = tmp[t];
  __syncthreads();
  return r;
}

// Largest index i in [0, n) with key(i) <= x, or -1.
template <typename F>
__device__ int last_le(int n, int64_t x, F key) {
  int lo = 0, hi = n;  // answer in [lo - 1, hi - 1]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (key(mid) <= x) lo = mid + 1; else hi = mid;
  }
  return lo - 1;
}

__global__ __launch_bounds__(kPlanThreads) void mla_plan_kernel(const int32_t* __restrict__ seqlens, char* ws,
                                                                Layout lay, int batch, int seqlen_q, int rows,
                                                                int nwg, int max_blocks) {
  __shared__ int64_t tmp[kPlanThreads];
  __shared__ int64_t carry_pages, carry_cost;
  __shared__ uint32_t flags;
  Header* hdr = reinterpret_cast<Header*>(ws + lay.header);
  WgInfo* wgi = reinterpret_cast<WgInfo*>(ws + lay.wg_info);
  ReqInfo* req = reinterpret_cast<ReqInfo*>(ws + lay.req_info);
  int64_t* cum_cost = reinterpret_cast<int64_t*>(ws + lay.cum_cost);
  int32_t* bounds = reinterpret_cast<int32_t*>(ws + lay.bounds);       // [nwg + 1]
  int32_t* ne_prefix = bounds + (nwg + 1);                              // [nwg + 1]
  const int t = threadIdx.x;
  const int64_t max_len = int64_t(max_blocks) * kPageSize;

  if (t == 0) { carry_pages = 0; carry_cost = 0; flags = 0; }
  __syncthreads();

  // 1. pages and cost per request; exclusive prefix sums of both.
  for (int base = 0; base < batch; base += kPlanThreads) {
    const int b = base + t;
    int64_t L = 0;
    if (b < batch) {
      L = seqlens[b];
      if (L < seqlen_q || L > max_len) atomicOr(&flags, 1u);
      L = L < 0 ? 0 : (L > max_len ? max_len : L);
    }
    const int64_t np = (L + kPageSize - 1) / kPageSize;
    const int64_t cost = np > 0 ? np + kPlanCostPerRequest : 0;
    const int64_t inc_p = block_inclusive_scan(np, tmp);
    const int64_t inc_c = block_inclusive_scan(cost, tmp);
    if (b < batch) {
      ReqInfo r;
      r.page_first = int32_t(carry_pages + inc_p - np);
      r.npages = int32_t(np);
      r.nsplit = 0;
      r.slot_off = 0;
      r.ne_lo = 0;
      r.seqlen = int32_t(L);
      r.pad0 = r.pad1 = 0;
      req[b] = r;
      cum_cost[b] = carry_cost + inc_c - cost;
    }
    __syncthreads();
    if (t == kPlanThreads - 1) { carry_pages += inc_p; carry_cost += inc_c; }
    __syncthreads();
  }
  const int64_t total_pages = carry_pages;
  const int64_t total_cost = carry_cost;
  if (t == 0) cum_cost[batch] = total_cost;
  __syncthreads();

  // 2. stretch boundaries in page positions: boundary s sits at cost s * T / nwg;
  //    a boundary inside a request's fixed-cost part moves to its first page.
  for (int s = t; s <= nwg; s += kPlanThreads) {
    int32_t bnd;
    if (s == nwg) {
      bnd = int32_t(total_pages);
    } else {
      const int64_t x = int64_t(s) * total_cost / nwg;
      const int b = last_le(batch, x, [&](int i) { return cum_cost[i]; });
      const int64_t off = x - cum_cost[b] - kPlanCostPerRequest;
      const int64_t np = req[b].npages;
      bnd = req[b].page_first + int32_t(off < 0 ? 0 : (off > np ? np : off));
    }
    bounds[s] = bnd;
  }
  __syncthreads();

  // 3. non-empty stretches: exclusive prefix count, then per-stretch info.
  {
    int64_t carry = 0;
    for (int base = 0; base <= nwg; base += kPlanThreads) {
      const int s = base + t;
      const int64_t ne = (s < nwg && bounds[s + 1] > bounds[s]) ? 1 : 0;
      const int64_t inc = block_inclusive_scan(ne, tmp);
      if (s <= nwg) ne_prefix[s] = int32_t(carry + inc - ne);
      __syncthreads();
      if (t == kPlanThreads - 1) tmp[0] = inc;
      __syncthreads();
      carry += tmp[0];
      __syncthreads();
    }
  }
  __syncthreads();
  for (int s = t; s < nwg; s += kPlanThreads) {
    WgInfo w;
    w.page_begin = bounds[s];
    w.page_end = bounds[s + 1];
    w.b_begin = w.page_begin < total_pages
                    ? last_le(batch, w.page_begin, [&](int i) { return (int64_t)req[i].page_first; })
                    : batch;
    w.ne_prefix = ne_prefix[s];
    wgi[s] = w;
  }
  __syncthreads();

  // 4. per request: how many stretches hold it, and its partial slots.
  {
    int64_t carry = 0;
    for (int base = 0; base < batch; base += kPlanThreads) {
      const int b = base + t;
      int nsplit = 0, ne_lo = 0;
      if (b < batch && req[b].npages > 0) {
        const int64_t first = req[b].page_first, end = first + req[b].npages;
        // first stretch whose end is past the request's first page
        const int s_lo = 1 + last_le(nwg, first, [&](int i) { return (int64_t)bounds[i + 1]; });
        // last stretch whose begin is before the request's end
        const int s_hi = last_le(nwg, end - 1, [&](int i) { return (int64_t)bounds[i]; });
        nsplit = ne_prefix[s_hi + 1] - ne_prefix[s_lo];
        ne_lo = ne_prefix[s_lo];
      }
      const int64_t slots = nsplit > 1 ? nsplit : 0;
      const int64_t inc = block_inclusive_scan(slots, tmp);
      if (b < batch) {
        req[b].nsplit = nsplit;
        req[b].ne_lo = ne_lo;
        req[b].slot_off = int32_t(carry + inc - slots);
      }
      __syncthreads();
      if (t == kPlanThreads - 1) tmp[0] = inc;
      __syncthreads();
      carry += tmp[0];
      __syncthreads();
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
      h.total_pages = int32_t(total_pages);
      h.used_slots = int32_t(carry);
      for (int i = 0; i < 7; i++) h.pad[i] = 0;
      *hdr = h;
    }
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
