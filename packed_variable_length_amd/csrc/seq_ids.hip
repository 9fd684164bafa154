// Per-token segment ids of a frame-padded pack, and the status strings.
//
// "LingBot-VA packing" report, section 2.1: every episode is zero-padded to the
// same frame count; the mask builder gives the tokens of frames at or past
// valid_frames[b] the id -1 and the other tokens of episode b the id b.
#include "pa_common.h"

namespace {

// One thread per output token; a grid-stride loop covers any size.  Token
// index t decomposes as ((b * frames_padded) + f) * tokens_per_frame + i.
__global__ void __launch_bounds__(256)
seq_ids_kernel(const int32_t* __restrict__ valid_frames, int32_t frames_padded,
               int32_t tokens_per_frame, int64_t n_tokens, int32_t* __restrict__ seq_id) {
  const int64_t per_episode = (int64_t)frames_padded * tokens_per_frame;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n_tokens;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int32_t b = (int32_t)(t / per_episode);
    const int32_t f = (int32_t)((t - (int64_t)b * per_episode) / tokens_per_frame);
    int32_t vf = valid_frames[b];
    vf = vf < 0 ? 0 : (vf > frames_padded ? frames_padded : vf);
    seq_id[t] = f < vf ? b : -1;
  }
}

}  // namespace

extern "C" const char* pa_status_str(int32_t s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: a size is out of range";
    case PA_ERR_DTYPE: return "PA_ERR_DTYPE: unknown dtype";
    case PA_ERR_HEADDIM: return "PA_ERR_HEADDIM: head_dim must be 64 or 128";
    case PA_ERR_MASK_MISMATCH: return "PA_ERR_MASK_MISMATCH: block mask does not fit this call";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: storage or workspace too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: a HIP launch failed";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN: pointer not 16-byte (storage: 256-byte) aligned";
    default: return "unknown status";
  }
}

extern "C" int32_t seq_ids_from_valid_frames(const int32_t* valid_frames, int32_t B,
                                             int32_t frames_padded, int32_t tokens_per_frame,
                                             int32_t* seq_id, void* stream) {
  if (B < 0 || frames_padded < 1 || tokens_per_frame < 1) return PA_ERR_SHAPE;
  const int64_t n = (int64_t)B * frames_padded * tokens_per_frame;
  if (n > INT32_MAX) return PA_ERR_SHAPE;
  if (n == 0) return PA_OK;
  if (!valid_frames || !seq_id) return PA_ERR_NULL;
  const int64_t blocks64 = (n + 255) / 256;
  const int blocks = (int)(blocks64 < 65536 ? blocks64 : 65536);
  hipLaunchKernelGGL(seq_ids_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     valid_frames, frames_padded, tokens_per_frame, n, seq_id);
  return pa::launch_status();
}
