"""Build-time scan of generated gfx950 assembly (not loaded at run time).

The library must write device memory only through the vector memory path;
this lists the scalar-cache write instructions and finds any in an .s file.
"""
SCALAR_CACHE_WRITES = ("s_store", "s_atomic", "s_dcache_wb", "s_buffer_store", "s_scratch_store")


def scalar_cache_writes(asm_text: str):
    return [line.strip() for line in asm_text.splitlines()
            if line.strip().startswith(SCALAR_CACHE_WRITES)]
