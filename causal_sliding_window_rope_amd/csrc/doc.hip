// Document segments of packed rows: per token the [start, end) of the maximal run of equal
// document ids that contains it ("从4万美元到73美元" §6.1: BOS-aligned rows packing several
// documents; attention stays inside a token's own document). Computed once per batch and
// shared by every layer's attention calls.
#include "common.h"
#include "internal.h"

namespace swa {

constexpr int kDocThreads = 1024;

// One workgroup per row b; thread i scans a contiguous chunk of the row. A run starts at t
// when t == 0 or ids[t] != ids[t-1]. start[t] = the last run start <= t (prefix max over
// chunks), end[t] = the first run start > t, or T (suffix min over chunks).
__global__ void __launch_bounds__(kDocThreads) doc_bounds_kernel(const int* __restrict__ ids,
                                                                 int* __restrict__ bounds, int T) {
  __shared__ int last_sc[kDocThreads], first_sc[kDocThreads];
  const int tid = threadIdx.x;
  const int* row = ids + (size_t)blockIdx.x * T;
  int* out = bounds + (size_t)blockIdx.x * T * 2;
  const int per = (T + kDocThreads - 1) / kDocThreads;
  const int t0 = min(T, tid * per), t1 = min(T, t0 + per);
  auto starts_run = [&](int t) { return t == 0 || row[t] != row[t - 1]; };
  int last = -1, first = T;
  for (int t = t0; t < t1; ++t) {
    if (starts_run(t)) {
      last = t;
      first = min(first, t);
    }
  }
  last_sc[tid] = last;
  first_sc[tid] = first;
  __syncthreads();
  // inclusive prefix max of `last`, inclusive suffix min of `first` (Hillis-Steele)
  for (int off = 1; off < kDocThreads; off <<= 1) {
    const int a = tid >= off ? last_sc[tid - off] : -1;
    const int c = tid + off < kDocThreads ? first_sc[tid + off] : T;
    __syncthreads();
    last_sc[tid] = max(last_sc[tid], a);
    first_sc[tid] = min(first_sc[tid], c);
    __syncthreads();
  }
  int run_start = tid > 0 ? last_sc[tid - 1] : -1;                  // last start before the chunk
  int run_next = tid + 1 < kDocThreads ? first_sc[tid + 1] : T;     // first start after it
  for (int t = t0; t < t1; ++t) {
    if (starts_run(t)) run_start = t;
    out[2 * t] = run_start;
  }
  for (int t = t1 - 1; t >= t0; --t) {
    out[2 * t + 1] = run_next;
    if (starts_run(t)) run_next = t;
  }
}

hipError_t launch_doc_bounds(const int* doc_id, int* bounds, int B, int T, hipStream_t s) {
  hipLaunchKernelGGL(doc_bounds_kernel, dim3(B), dim3(kDocThreads), 0, s, doc_id, bounds, T);
  return hipGetLastError();
}

}  // namespace swa
