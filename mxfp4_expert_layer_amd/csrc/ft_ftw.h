// FTW expert files inside libft: the reader the disk tier of the miss path uses.
#pragma once

#include "ft_host.h"

namespace ft {

// The host thread pool of a context (null for a null context).
ThreadPool* ctx_pool(ft_ctx* ctx);

// Read blobs ids[0..n-1] of f into dst[i], in requests of `chunk` bytes (0: whole blobs),
// over the pool's threads (pool may be null).  Checks ids and O_DIRECT alignment.
int ftw_read(ThreadPool* pool, ft_ftw* f, const int32_t* ids, int n, uint8_t* const* dst,
             uint64_t chunk);
uint64_t ftw_blob_stride(const ft_ftw* f);
void ftw_dims(const ft_ftw* f, int* fmt, int* H, int* I, int* E, int* n_shared);

}  // namespace ft
