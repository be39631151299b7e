// GPU-built, cost-sorted tile lists (FLAMIA paper, Section 3.6.2 and
// Appendix B.6): built on the device in one single-workgroup launch, no
// host synchronization.
//
// A document of L tokens has n = ceil(L/128) tiles of 128 tokens, anchored at
// its first token.
//   query-major (forward, dQ): query tile t attends t+1 key tiles  -> cost t + 1
//   key-major (dK/dV)        : key tile t meets n - t query tiles  -> cost n - t
// Both give every document the costs 1..n, so one histogram serves both.
// Tiles are ordered by decreasing cost (longest first; the hardware
// dispatches workgroups in index order, so the expensive items start first
// and the cheap ones fill in at the end).  Sorting is a counting sort on the
// small integer cost instead of a comparison sort.  Within one cost class the
// order is whatever the atomics give; it does not change any result.
// Work item (tile, head) is decoded by the attention kernels from the
// workgroup index, heads innermost.
//
// ctrl layout (int32): [0] number of tiles, [1] 1 if the backward's dS store
// holds this call's blocks (capacity given and not exceeded), else 0,
// [16, 16+C1) query-major cursors, [16+C1, 16+2 C1) key-major cursors
// (C1 = max_cost + 1).  The dS block offsets of the documents go to dboff.
#include "device.h"
#include "kernels.h"

namespace flamia {

constexpr int kPlanThreads = 1024;

// In-place inclusive scan of buf[0..n) in LDS by a 1024-thread block;
// reverse = true scans from the end (suffix sums).
__device__ void block_scan(int* buf, int n, bool reverse, int* partial) {
    const int tid = threadIdx.x;
    const int chunk = (n + kPlanThreads - 1) / kPlanThreads;
    const int lo = tid * chunk, hi = min(lo + chunk, n);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += buf[reverse ? n - 1 - i : i];
    partial[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        const int v = tid >= off ? partial[tid - off] : 0;
        __syncthreads();
        partial[tid] += v;
        __syncthreads();
    }
    int run = tid > 0 ? partial[tid - 1] : 0;
    for (int i = lo; i < hi; ++i) {
        const int j = reverse ? n - 1 - i : i;
        run += buf[j];
        buf[j] = run;
    }
    __syncthreads();
}

__global__ void __launch_bounds__(kPlanThreads)
plan_kernel(const int32_t* __restrict__ cu, int ndocs, int max_cost, int32_t* __restrict__ tiles_prefix,
            int32_t* __restrict__ ctrl, long max_tiles, int4* __restrict__ tiles_q, int4* __restrict__ tiles_k,
            int32_t* __restrict__ dboff, long ds_blocks) {
    extern __shared__ int smem[];
    int* partial = smem;                       // kPlanThreads
    int* hist = smem + kPlanThreads;           // max_cost + 1
    const int tid = threadIdx.x;
    const int C1 = max_cost + 1;
    for (int c = tid; c < C1; c += kPlanThreads) hist[c] = 0;
    __syncthreads();
    for (int d = tid; d < ndocs; d += kPlanThreads) {
        const int L = cu[d + 1] - cu[d];
        const int n = min((L + kTile - 1) / kTile, max_cost);
        if (n > 0) atomicAdd(&hist[n], 1);
    }
    __syncthreads();
    // hist[c] = #docs with n >= c = number of tiles of cost c (c >= 1)
    block_scan(hist, C1, true, partial);
    // hist[c] = number of tiles of cost >= c; the class of cost c starts at
    // hist[c + 1] (classes by decreasing cost) and hist[1] is the total
    block_scan(hist, C1, true, partial);
    const int total = C1 > 1 ? (int)min((long)hist[1], max_tiles) : 0;
    for (int c = tid; c < C1; c += kPlanThreads) {
        ctrl[16 + c] = 0;                      // query-major cursors
        ctrl[16 + C1 + c] = 0;                 // key-major cursors
    }
    if (tid == 0) ctrl[0] = total;
    // exclusive prefix of tile counts over documents
    {
        const int chunk = (ndocs + kPlanThreads - 1) / kPlanThreads;
        const int lo = tid * chunk, hi = min(lo + chunk, ndocs);
        int sum = 0;
        for (int d = lo; d < hi; ++d) sum += (cu[d + 1] - cu[d] + kTile - 1) / kTile;
        partial[tid] = sum;
        __syncthreads();
        for (int o = 1; o < kPlanThreads; o <<= 1) {
            const int v = tid >= o ? partial[tid - o] : 0;
            __syncthreads();
            partial[tid] += v;
            __syncthreads();
        }
        int run = tid > 0 ? partial[tid - 1] : 0;
        for (int d = lo; d < hi; ++d) {
            tiles_prefix[d] = run;
            run += (cu[d + 1] - cu[d] + kTile - 1) / kTile;
        }
        if (tid == kPlanThreads - 1) tiles_prefix[ndocs] = partial[kPlanThreads - 1];
    }
    // dS store: first causal 32x32 block of each document (nb (nb + 1) / 2
    // blocks for nb = ceil(L / 32)), and whether the call fits the capacity
    if (dboff) {
        __syncthreads();
        const int chunk = (ndocs + kPlanThreads - 1) / kPlanThreads;
        const int lo = tid * chunk, hi = min(lo + chunk, ndocs);
        long sum = 0;
        for (int d = lo; d < hi; ++d) {
            const long nb = (cu[d + 1] - cu[d] + kBlock - 1) / kBlock;
            sum += nb * (nb + 1) / 2;
        }
        __shared__ long lpartial[kPlanThreads];
        lpartial[tid] = sum;
        __syncthreads();
        for (int o = 1; o < kPlanThreads; o <<= 1) {
            const long v = tid >= o ? lpartial[tid - o] : 0;
            __syncthreads();
            lpartial[tid] += v;
            __syncthreads();
        }
        const long total_blocks = lpartial[kPlanThreads - 1];
        const bool fits = ds_blocks > 0 && total_blocks <= ds_blocks;
        long run = tid > 0 ? lpartial[tid - 1] : 0;
        for (int d = lo; d < hi; ++d) {
            dboff[d] = fits ? (int32_t)run : 0;
            const long nb = (cu[d + 1] - cu[d] + kBlock - 1) / kBlock;
            run += nb * (nb + 1) / 2;
        }
        if (tid == 0) ctrl[1] = fits ? 1 : 0;
    } else if (tid == 0) {
        ctrl[1] = 0;
    }
    // the cursor zeros and the prefix table must have reached L2 before any
    // thread of the workgroup uses them
    __threadfence();
    __syncthreads();
    for (int p = tid; p < total; p += kPlanThreads) {
        const int doc = find_doc(tiles_prefix, ndocs, p);
        const int t = p - tiles_prefix[doc];
        const int n = tiles_prefix[doc + 1] - tiles_prefix[doc];
        const int ds = cu[doc], de = cu[doc + 1];
        const int4 tile = make_int4(ds + kTile * t, ds, de, doc);
        {
            const int cost = t + 1;
            const int slot = (cost + 1 < C1 ? hist[cost + 1] : 0) + atomicAdd(&ctrl[16 + cost], 1);
            if (slot < max_tiles) tiles_q[slot] = tile;
        }
        if (tiles_k) {
            const int cost = n - t;
            const int slot = (cost + 1 < C1 ? hist[cost + 1] : 0) + atomicAdd(&ctrl[16 + C1 + cost], 1);
            if (slot < max_tiles) tiles_k[slot] = tile;
        }
    }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t st) {
    const size_t smem = sizeof(int) * (kPlanThreads + a.max_cost + 1);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), smem, st, a.cu, a.ndocs, a.max_cost,
                       a.tiles_prefix, a.ctrl, a.max_tiles, a.tiles_q, a.tiles_k, a.dboff, a.ds_blocks);
    return hipGetLastError();
}

}  // namespace flamia
