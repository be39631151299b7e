// GPU-built, cost-sorted work lists (FLAMIA paper, Section 3.6.2 and
// Appendix B.6): built once per call on the device, no host synchronization,
// a fixed number of launches.
//
// A tile item is (document, 128-token tile t, head).  A document of L tokens
// has n = ceil(L/128) tiles, anchored at its first token.
//   forward : query tile t attends t+1 key tiles      -> cost t + 1
//   backward: key tile t meets n - t query tiles      -> cost n - t
// Both give every document the costs 1..n, so one histogram serves both.
// Items are ordered by decreasing cost (longest first; the hardware dispatches
// workgroups in index order, so the expensive items start first and the
// cheap ones fill in at the end).  Sorting is a counting sort on the small
// integer cost instead of a comparison sort.  Within one cost class the order
// is whatever the atomics give; it does not change any result.
//
// ctrl layout (int32): [0] query-major item count, [1] tile count,
//   [2] key-major item count, [16, 16+C1) offset of each cost class,
//   [16+C1, 16+2 C1) query-major cursors, [16+2 C1, 16+3 C1) key-major cursors
//   (C1 = max_cost + 1).
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
plan_count_kernel(const int32_t* __restrict__ cu, int ndocs, int max_cost,
                  int32_t* __restrict__ tiles_prefix, int32_t* __restrict__ ctrl, int heads_q, int heads_k) {
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
    block_scan(hist, C1, true, partial);       // hist[c] = #docs with n >= c = items of cost c
    int* cnt = hist;
    // offsets: classes ordered by decreasing cost -> exclusive suffix sum
    for (int c = tid; c < C1; c += kPlanThreads) ctrl[16 + c] = cnt[c];
    __syncthreads();
    // exclusive suffix of cnt over c >= 1, in place in LDS (hist reused)
    for (int c = tid; c < C1; c += kPlanThreads) hist[c] = c >= 1 ? ctrl[16 + c] : 0;
    __syncthreads();
    block_scan(hist, C1, true, partial);       // inclusive suffix
    for (int c = tid; c < C1; c += kPlanThreads) {
        const int incl = hist[c];
        const int own = c >= 1 ? ctrl[16 + c] : 0;
        ctrl[16 + c] = incl - own;             // exclusive: sum over c' > c
        ctrl[16 + C1 + c] = 0;                 // cursors
        ctrl[16 + 2 * C1 + c] = 0;
    }
    if (tid == 0) {
        ctrl[1] = hist[1];                     // all tiles
        ctrl[0] = hist[1] * heads_q;
        ctrl[2] = hist[1] * heads_k;
    }
    __syncthreads();
    // exclusive prefix of tile counts over documents
    // (chunked over the documents; reuses `hist` as a staging buffer of kPlanThreads)
    {
        const int chunk = (ndocs + kPlanThreads - 1) / kPlanThreads;
        const int lo = tid * chunk, hi = min(lo + chunk, ndocs);
        int sum = 0;
        for (int d = lo; d < hi; ++d) sum += (cu[d + 1] - cu[d] + kTile - 1) / kTile;
        partial[tid] = sum;
        __syncthreads();
        for (int off = 1; off < kPlanThreads; off <<= 1) {
            const int v = tid >= off ? partial[tid - off] : 0;
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
}

__global__ void __launch_bounds__(256)
plan_fill_kernel(const int32_t* __restrict__ cu, int ndocs, int max_cost,
                 const int32_t* __restrict__ tiles_prefix, int32_t* __restrict__ ctrl, long max_tiles,
                 int heads_q, int4* __restrict__ items_q, int heads_k, int4* __restrict__ items_k) {
    const long p = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const int total = ctrl[1];
    if (p >= total || p >= max_tiles) return;
    const int doc = find_doc(tiles_prefix, ndocs, (int)p);
    const int t = (int)p - tiles_prefix[doc];
    const int n = tiles_prefix[doc + 1] - tiles_prefix[doc];
    const int C1 = max_cost + 1;
    const int ds = cu[doc], de = cu[doc + 1];
    {
        const int cost = t + 1;
        const int slot = ctrl[16 + cost] + atomicAdd(&ctrl[16 + C1 + cost], 1);
        for (int h = 0; h < heads_q; ++h) items_q[(long)slot * heads_q + h] = make_int4(ds + kTile * t, ds, de, h);
    }
    if (items_k) {
        const int cost = n - t;
        const int slot = ctrl[16 + cost] + atomicAdd(&ctrl[16 + 2 * C1 + cost], 1);
        for (int h = 0; h < heads_k; ++h) items_k[(long)slot * heads_k + h] = make_int4(ds + kTile * t, ds, de, h);
    }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t st) {
    const size_t smem = sizeof(int) * (kPlanThreads + a.max_cost + 1);
    hipLaunchKernelGGL(plan_count_kernel, dim3(1), dim3(kPlanThreads), smem, st, a.cu, a.ndocs, a.max_cost,
                       a.tiles_prefix, a.ctrl, a.heads_q, a.items_k ? a.heads_k : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned blocks = (unsigned)((a.max_tiles + 255) / 256);
    hipLaunchKernelGGL(plan_fill_kernel, dim3(blocks), dim3(256), 0, st, a.cu, a.ndocs, a.max_cost,
                       a.tiles_prefix, a.ctrl, a.max_tiles, a.heads_q, a.items_q, a.heads_k, a.items_k);
    return hipGetLastError();
}

}  // namespace flamia
