// Device-side check of the caller's device-resident index data: the sequence lengths, the block table
// and the prefill chunk offsets. The host cannot read them before a launch, and the append and
// attention kernels trust them to stay inside the cache ("论文复现工坊 No.4", section 2: the cache is
// addressed by sequence and position; the paged layout of the cache descriptor adds the block table).
// One work-group reads only those arrays, never the cache, and writes a bit mask of the rules the data
// breaks (0: none), so a caller can test suspicious inputs before handing them to the other kernels.
#include "mla_internal.h"

namespace mla {

__global__ void __launch_bounds__(256) check_inputs_kernel(int batch, const int32_t* __restrict__ seq_lens,
                                                           const int32_t* __restrict__ table, int max_blocks,
                                                           int64_t num_blocks, int block_size,
                                                           const int32_t* __restrict__ cu_q_lens, int total_q,
                                                           int32_t* __restrict__ error_word) {
  __shared__ int flags;
  if (threadIdx.x == 0) flags = 0;
  __syncthreads();
  int f = 0;
  const int64_t cap = (int64_t)max_blocks * block_size;
  for (int b = threadIdx.x; b < batch; b += blockDim.x) {
    const int len = seq_lens[b];
    if (len < 0 || len > cap) f |= kCheckBadLength;
    if (cu_q_lens != nullptr) {
      const int c0 = cu_q_lens[b], c1 = cu_q_lens[b + 1];
      if (c1 < c0)
        f |= kCheckBadOffsets;
      else if (len >= 0 && c1 - c0 > len)
        f |= kCheckChunkTooLong;
    }
  }
  if (cu_q_lens != nullptr && threadIdx.x == 0 && (cu_q_lens[0] != 0 || cu_q_lens[batch] != total_q))
    f |= kCheckBadOffsets;
  // logical block i of sequence b is used when i < ceil(len_b / block_size), len_b clamped to the capacity
  const int64_t items = (int64_t)batch * max_blocks;
  for (int64_t it = threadIdx.x; it < items; it += blockDim.x) {
    const int b = (int)(it / max_blocks), i = (int)(it % max_blocks);
    const int64_t len = min<int64_t>(max<int64_t>(seq_lens[b], 0), cap);
    if ((int64_t)i * block_size >= len) continue;
    const int64_t phys = table != nullptr ? (int64_t)table[it] : it;
    if (phys < 0 || phys >= num_blocks) f |= kCheckBadBlock;
  }
  if (f != 0) atomicOr(&flags, f);
  __syncthreads();
  if (threadIdx.x == 0) *error_word = flags;
}

hipError_t launch_check_inputs(int batch, const int32_t* seq_lens, const int32_t* table, int max_blocks,
                               int64_t num_blocks, int block_size, const int32_t* cu_q_lens, int total_q,
                               int32_t* error_word, hipStream_t stream) {
  hipLaunchKernelGGL(check_inputs_kernel, dim3(1), dim3(256), 0, stream, batch, seq_lens, table, max_blocks, num_blocks,
                     block_size, cu_q_lens, total_q, error_word);
  return hipGetLastError();
}

}  // namespace mla
