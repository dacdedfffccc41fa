// Internal interface between the C-ABI front end (kda_api.cpp, plain C++)
// and the HIP translation units that hold the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace kda {

// Bytes of workspace one (chunk, head) needs, per element type and width.
// Returns 0 for an unsupported combination.
size_t chunk_bytes(int is_bf16, int d);

// Enqueue the chunked forward.  All arguments were validated by the caller.
// n_seq_rows: number of sequences (n_seqs, or B when cu == nullptr);
// n_chunks: upper bound of chunks over all sequences.  Returns a hipError_t.
int launch_chunk_forward(int is_bf16, int d, int n_seq_rows, int T, int H,
                         int64_t n_chunks, float g_floor, const void* q,
                         const void* k, const void* v, const void* g,
                         const float* beta, const float* h0,
                         const int32_t* cu, void* o, float* ht, void* ws,
                         void* stream);

// Enqueue one decode step.  Returns a hipError_t.
int launch_decode_step(int is_bf16, int d, int N, int H, float g_floor,
                       const void* q, const void* k, const void* v,
                       const void* g, const float* beta, float* state, void* o,
                       void* stream);

}  // namespace kda
