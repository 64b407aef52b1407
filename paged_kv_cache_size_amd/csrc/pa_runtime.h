// Host-side runtime queries shared by the libpa launchers (HIP calls, cached
// per device where they cost a driver round trip), and the one launcher one
// source file lends another.
#pragma once

#include <stdint.h>

namespace pa {

// Compute units of the current device, or -1.
int device_cu_count();
// Workgroups of kernel `fn` with `threads` threads that fit one compute unit
// at once (cached per device and kernel), or 0 on failure.
int resident_per_cu(const void* fn, int threads);
// PA_OK, or PA_ERR_HIP if the last launch failed.
int launch_status();

struct DecodeShape;
struct PoolView;
// The VALU decode kernel run over the query rows of a varlen batch (fp32
// prefill): the kernel for shape `s` (num_seqs = sequences) and its
// workgroup size, then the launch over `num_rows` rows (query_start_loc [num_seqs + 1]),
// partials into ws_acc [rows, H, parts, D] / ws_ml [rows, H, parts] when a
// row's keys span several partitions.
const void* decode_rows_kernel(const DecodeShape& s, int* threads);
int launch_decode_rows(void* out, const void* query, const PoolView& pv, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* query_start_loc, const DecodeShape& s,
                       int num_rows, float scale, void* ws_acc, void* ws_ml, int part_tokens, int num_parts,
                       void* stream);

}  // namespace pa
