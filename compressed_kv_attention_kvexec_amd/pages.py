"""Host page allocator of libtq4.so (tq4_pages_* in include/tq4.h): marshalling only."""
from __future__ import annotations

import ctypes

from ._binding import TQ4_ERR_CAPACITY, Tq4Error, check, load_library


class PageAllocator:
    """Page IDs for the TQ4 pools: admission reservations, shared-prefix reference counts and
    release at the step boundary, all in the C library."""

    def __init__(self, num_pages: int, page_size: int):
        self._lib = load_library()
        self._h = ctypes.c_void_p()
        check(self._lib.tq4_pages_create(num_pages, page_size, ctypes.byref(self._h)))
        self.num_pages, self.page_size = num_pages, page_size

    def close(self) -> None:
        if self._h:
            self._lib.tq4_pages_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        self.close()

    @staticmethod
    def admission_need(prompt_len: int, output_budget: int, page_size: int) -> int:
        return int(load_library().tq4_pages_admission_need(prompt_len, output_budget, page_size))

    def admit(self, prompt_len: int, output_budget: int, prefix_pages=()) -> int | None:
        """The request handle, or None when the reservation does not fit."""
        pre = (ctypes.c_int32 * max(len(prefix_pages), 1))(*prefix_pages)
        rid = ctypes.c_int32(-1)
        st = self._lib.tq4_pages_admit(self._h, prompt_len, output_budget, pre, len(prefix_pages), ctypes.byref(rid))
        if st == TQ4_ERR_CAPACITY:
            return None
        check(st)
        return rid.value

    def extend(self, request: int, length: int) -> bool:
        """False (nothing changes) when too few pages are free."""
        st = self._lib.tq4_pages_extend(self._h, request, length)
        if st == TQ4_ERR_CAPACITY:
            return False
        check(st)
        return True

    def table(self, request: int) -> list[int]:
        n = self._lib.tq4_pages_table(self._h, request, None, 0)
        if n < 0:
            raise Tq4Error(2, "bad request handle")
        buf = (ctypes.c_int32 * max(n, 1))()
        self._lib.tq4_pages_table(self._h, request, buf, n)
        return list(buf[:n])

    def finish(self, request: int) -> None:
        check(self._lib.tq4_pages_finish(self._h, request))

    def boundary(self) -> None:
        check(self._lib.tq4_pages_boundary(self._h))

    def free_list(self) -> list[int]:
        n = self._lib.tq4_pages_free_list(self._h, None, 0)
        buf = (ctypes.c_int32 * max(n, 1))()
        self._lib.tq4_pages_free_list(self._h, buf, n)
        return list(buf[:n])

    def refcount(self, page: int) -> int:
        return int(self._lib.tq4_pages_refcount(self._h, page))

    def reserved(self) -> int:
        return int(self._lib.tq4_pages_reserved(self._h))
