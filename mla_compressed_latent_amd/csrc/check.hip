// The check of device-resident arguments run by the checking build of the
// library (MLA_DEBUG_CHECKS): one workgroup walks the sequences with the
// functions of check.hpp and writes the first failure.
#include "check.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

constexpr int kCheckThreads = 256;

// result[0]: kNone or encode(b, code) of the lowest failing sequence b;
// result[1]: that failure's detail value.  Every thread takes the sequences
// b = tid, tid + 256, ... and keeps its own first failure; the minimum over
// threads (an LDS atomic) is the lowest failing sequence of all.
__global__ __launch_bounds__(kCheckThreads) void check_args_kernel(
    int append, const int32_t* cu, const int32_t* lens, const int32_t* page_table, int max_pages, int batch,
    int total, int max_q_len, int max_seq_len, int page_size, int64_t num_pages, uint32_t* result) {
  __shared__ uint32_t first;
  __shared__ int32_t first_detail;
  if (threadIdx.x == 0) {
    first = mla_check::kNone;
    first_detail = 0;
  }
  __syncthreads();
  uint32_t mine = mla_check::kNone;
  int32_t mine_detail = 0;
  for (int b = threadIdx.x; b < batch && mine == mla_check::kNone; b += kCheckThreads) {
    int32_t detail = 0;
    const uint32_t code =
        append ? mla_check::check_append_sequence(b, cu, lens, page_table, max_pages, batch, total, page_size,
                                                  num_pages, &detail)
               : mla_check::check_decode_sequence(b, cu, lens, page_table, max_pages, batch, total, max_q_len,
                                                  max_seq_len, page_size, num_pages, &detail);
    if (code != mla_check::kOk) {
      mine = mla_check::encode(b, code);
      mine_detail = detail;
    }
  }
  if (mine != mla_check::kNone) atomicMin(&first, mine);
  __syncthreads();
  if (mine != mla_check::kNone && mine == first) first_detail = mine_detail;
  __syncthreads();
  if (threadIdx.x == 0) {
    result[0] = first;
    result[1] = (uint32_t)first_detail;
  }
}

}  // namespace

void launch_check_args(bool append, const int32_t* cu, const int32_t* lens, const int32_t* page_table,
                       int max_pages, int batch, int total, int max_q_len, int max_seq_len, int page_size,
                       int64_t num_pages, uint32_t* result, hipStream_t st) {
  hipLaunchKernelGGL(check_args_kernel, dim3(1), dim3(kCheckThreads), 0, st, append ? 1 : 0, cu, lens,
                     page_table, max_pages, batch, total, max_q_len, max_seq_len, page_size, num_pages, result);
}

}  // namespace mla
